// Paged KV-cache decode attention for MI355X (gfx950, CDNA4, wave64).
//
// Three kernels:
//   pa_cache_write_kernel  -- scatter each new token's K/V row into its slot.
//   pa_partition_kernel    -- attention of one (sequence, kv head, query-head tile,
//                             context partition) over the paged K/V.
//   pa_reduce_kernel       -- log-sum-exp merge of a sequence's partitions.
//
// Sources (page title, section):
//  [DRV]  "揭开 NVIDIA 驱动栈的面纱：GPU 显存页表与 vLLM 中的 PagedAttention 是如何在底层协同的"
//         (kwkd.cn), section 6: block table lookup of a logical position and the
//         block * block-stride + head * head-stride + offset address of a K row.
//  [SRC]  vLLM source walk-through (peacm.com), section 3.2 (append into the last
//         block), section 3.4 (loop over logical blocks, tail mask, online softmax).
//  [CON]  "PagedAttention：当 KV Cache 遇到操作系统分页" (forceinjection.github.io),
//         section 3.2 (the kernel walks the table block by block); section 5.1 (keep
//         the table slice in fast memory to hide the software translation).
//  [SOSP] "《Efficient Memory Management for LLM Serving with PagedAttention》深度解读报告"
//         (zako-mio.github.io), sections 2.3 and 3.3 (only the filled slots of a block
//         take part; the result equals attention over contiguous K/V).
//
// Design for gfx950 (not a translation of the pages' CUDA kernel):
//  * The pool layout [N, Hkv, B, D] makes one (block, kv head) tile a contiguous
//    B*D run, so a wave reads it with 16-byte loads whose lanes cover whole rows.
//  * All G query heads that share a kv head are handled by one work-group, so each
//    K/V tile is read from HBM once per group (GQA), not once per query head.
//  * K pass: C lanes share one token row; each multiplies its 16-byte chunks with
//    the matching q chunks (v_dot2 for fp16), and the C partial sums are combined
//    with DPP row permutations fused into the adds.  Scores go to LDS.
//  * Softmax: one wave per query row takes the chunk max and exp-sum with wave
//    shuffles; the running max and sum carry over chunks (online softmax, [SRC] 3.4).
//  * V pass: a whole 16-byte chunk per lane (CV lanes per row), fp32 accumulators.
//  * Contexts are split into partitions (split-K) so that short batches still fill
//    256 CUs; a second kernel merges them in partition order.
//  * Every reduction runs in a fixed order that depends only on logical positions,
//    so results are bitwise reproducible under any physical block placement.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "pa.h"

namespace {

using f16 = _Float16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWaves = 4;                 // waves per decode work-group
constexpr int kThreads = kWaves * kWave;  // 256
constexpr int kChunk = 512;               // tokens whose scores are held in LDS at once
constexpr int kMinBlock = 8;              // smallest supported block size

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of C consecutive lanes (C <= 16); every lane of the group
// ends with the same value.  Steps: swap neighbours, swap pairs (quad_perm), then
// mirror within 8 and within 16 lanes, which pair each lane with one in the other half.
template <int C>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(C == 1 || C == 2 || C == 4 || C == 8 || C == 16, "group width");
  if constexpr (C >= 2) x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (C >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (C >= 8) x += dpp_f<0x141>(x);  // row_half_mirror
  if constexpr (C >= 16) x += dpp_f<0x140>(x); // row_mirror
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = kWave / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Vector elements are copied to a scalar before reinterpretation: a bit cast applied
// directly to a subscripted vector element reads element 0 for every subscript.
template <typename To>
__device__ __forceinline__ To word_as(const u32x4& v, int i) {
  const uint32_t w = v[i];
  return __builtin_bit_cast(To, w);
}

// q-chunk . k-chunk over one 16-byte chunk, accumulated into acc.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float acc);

template <>
__device__ __forceinline__ float dot16<f16>(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2(word_as<f16x2>(a, i), word_as<f16x2>(b, i), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot16<float>(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(word_as<float>(a, i), word_as<float>(b, i), acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& v, float* f);

template <>
__device__ __forceinline__ void unpack16<f16>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = word_as<f16x2>(v, i);
    f[2 * i] = static_cast<float>(h.x);
    f[2 * i + 1] = static_cast<float>(h.y);
  }
}

template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = word_as<float>(v, i);
}

// Lanes per token row in the K pass: enough that the q chunks a lane keeps in
// registers stay near 32 VGPRs (64 for 8-row tiles), never fewer than a quarter
// of a row's 16-byte chunks, never more than all of them.
constexpr int pick_k_lanes(int row_bytes, int gt) {
  int cv = row_bytes / 16;
  int c = row_bytes * gt / 128;
  if (gt >= 8) c /= 2;
  if (c < cv / 4) c = cv / 4;
  if (c > cv) c = cv;
  if (c < 1) c = 1;
  return c;
}

template <typename T, int D, int GT>
struct Cfg {
  static constexpr int kRow = D * static_cast<int>(sizeof(T));  // bytes per token row
  static constexpr int kE = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
  static constexpr int kCV = kRow / 16;                         // lanes per row, V pass
  static constexpr int kC = pick_k_lanes(kRow, GT);             // lanes per row, K pass
  static constexpr int kNLK = kRow / (16 * kC);                 // chunks per lane per row, K pass
  static constexpr int kRK = kNLK >= 8 ? 1 : 8 / kNLK;          // rows per lane per K step
  static constexpr int kTK = kRK * (kWave / kC);                // tokens per wave per K step
  static constexpr int kRV = 8;                                 // rows per lane per V step
  static constexpr int kTV = kRV * (kWave / kCV);               // tokens per wave per V step
  static constexpr int kLds = (kChunk * GT > kWaves * GT * D) ? kChunk * GT : kWaves * GT * D;
  static_assert(kChunk % kTK == 0 && kChunk % kTV == 0, "chunk must hold whole steps");
  static_assert(kC <= 16, "K-pass group wider than one DPP row");
};

// ---------------------------------------------------------------------------
// cache write: one thread per 16-byte chunk of one (token, kv head) row
// ---------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void pa_cache_write_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int64_t* __restrict__ slot_mapping,
    T* __restrict__ k_cache, T* __restrict__ v_cache, int64_t num_chunks, int num_kv_heads,
    int block_size, int64_t num_slots) {
  constexpr int kChunksPerRow = D * static_cast<int>(sizeof(T)) / 16;
  constexpr int kE = 16 / static_cast<int>(sizeof(T));
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= num_chunks) return;
  const int c = static_cast<int>(i % kChunksPerRow);
  const int64_t row = i / kChunksPerRow;  // = t * Hkv + h
  const int h = static_cast<int>(row % num_kv_heads);
  const int64_t t = row / num_kv_heads;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * D + c * kE;
  const int64_t src = row * D + c * kE;
  *reinterpret_cast<u32x4*>(k_cache + dst) = load16(k + src);
  *reinterpret_cast<u32x4*>(v_cache + dst) = load16(v + src);
}

// ---------------------------------------------------------------------------
// decode, pass 1: one work-group per (partition, kv head x q-head tile, sequence)
// ---------------------------------------------------------------------------

struct PartitionArgs {
  void* out;
  float* ws_m;  // [S, Hq, max_parts]  running max of each partition (log2 units)
  float* ws_l;  // [S, Hq, max_parts]  exp-sum of each partition
  float* ws_o;  // [S, Hq, max_parts, D] normalised output of each partition
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;  // scale * log2(e): scores live in log2 units so exp2 is v_exp_f32
  int block_size;
  int log2_block;
  int num_kv_heads;
  int num_q_heads;
  int group;       // query heads per kv head
  int n_gtiles;    // ceil(group / GT)
  int max_blocks_per_seq;
  int max_context_len;
  int64_t num_blocks;
  int partition_size;
  int max_parts;
};

template <typename T, int D, int GT>
__global__ __launch_bounds__(kThreads) void pa_partition_kernel(const PartitionArgs a) {
  using K = Cfg<T, D, GT>;
  __shared__ float s_buf[K::kLds];              // scores, then probabilities, then partial sums
  __shared__ int s_tbl[kChunk / kMinBlock];     // physical ids of the chunk's blocks (-1 = invalid)
  __shared__ float s_m[GT], s_l[GT], s_corr[GT];
  __shared__ int s_bad;

  const int part = blockIdx.x;
  const int kvh = blockIdx.y / a.n_gtiles;
  const int gtile = blockIdx.y - kvh * a.n_gtiles;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;

  const int ctx = a.context_lens[s];
  const bool bad_ctx = ctx < 0 || ctx > a.max_context_len;
  const int nparts = (bad_ctx || ctx == 0) ? 1 : (ctx + a.partition_size - 1) / a.partition_size;
  if (part >= nparts) return;

  const int h0 = kvh * a.group + gtile * GT;
  const int ng = min(GT, a.group - gtile * GT);  // real rows in this tile
  const int64_t row0 = static_cast<int64_t>(s) * a.num_q_heads + h0;
  T* out = static_cast<T*>(a.out);

  if (bad_ctx || ctx == 0) {  // nothing to attend over: zeros, or NaN for an invalid length
    const T fill = static_cast<T>(bad_ctx ? __builtin_nanf("") : 0.0f);
    for (int i = tid; i < ng * D; i += kThreads) out[row0 * D + i] = fill;
    return;
  }

  const int t_begin = part * a.partition_size;
  const int t_end = min(ctx, t_begin + a.partition_size);

  // q chunks for the K pass: lane sub holds row chunks j*C + sub (j < NLK).
  const int subk = lane % K::kC;
  const T* qp = static_cast<const T*>(a.q);
  u32x4 qk[GT][K::kNLK];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int j = 0; j < K::kNLK; ++j)
      qk[g][j] = (g < ng) ? load16(qp + (row0 + g) * D + (j * K::kC + subk) * K::kE)
                          : u32x4{0u, 0u, 0u, 0u};

  if (tid == 0) s_bad = 0;
  if (tid < GT) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.0f;
  }

  float acc[GT][K::kE];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < K::kE; ++e) acc[g][e] = 0.0f;

  const int32_t* tbl_row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const int64_t head_stride = static_cast<int64_t>(a.block_size) * D;  // elements
  const int64_t block_stride = head_stride * a.num_kv_heads;
  const T* kbase = static_cast<const T*>(a.k_cache) + kvh * head_stride;
  const T* vbase = static_cast<const T*>(a.v_cache) + kvh * head_stride;
  const int bmask = a.block_size - 1;
  const int subv = lane % K::kCV;

  for (int c0 = t_begin; c0 < t_end; c0 += kChunk) {
    const int n = min(kChunk, t_end - c0);
    const int b0 = c0 >> a.log2_block;  // c0 is a multiple of the block size
    const int nb = (n + bmask) >> a.log2_block;
    __syncthreads();  // the previous chunk is done with s_tbl and s_buf
    for (int i = tid; i < nb; i += kThreads) {
      const int phys = tbl_row[b0 + i];
      s_tbl[i] = (phys < 0 || phys >= a.num_blocks) ? -1 : phys;
    }
    __syncthreads();

    // ---- K pass: scores of every query row for every token of the chunk
    for (int tile = w; tile * K::kTK < n; tile += kWaves) {
      u32x4 kr[K::kRK][K::kNLK];
#pragma unroll
      for (int r = 0; r < K::kRK; ++r) {
        const int tok = tile * K::kTK + r * (kWave / K::kC) + lane / K::kC;
        int phys = (tok < n) ? s_tbl[tok >> a.log2_block] : 0;
        if (phys < 0) {  // invalid table entry inside the context: poison, read block 0
          s_bad = 1;
          phys = 0;
        }
        const T* p = kbase + phys * block_stride + static_cast<int64_t>(tok & bmask) * D;
#pragma unroll
        for (int j = 0; j < K::kNLK; ++j) kr[r][j] = load16(p + (j * K::kC + subk) * K::kE);
      }
#pragma unroll
      for (int r = 0; r < K::kRK; ++r) {
        const int tok = tile * K::kTK + r * (kWave / K::kC) + lane / K::kC;
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          float d = 0.0f;
#pragma unroll
          for (int j = 0; j < K::kNLK; ++j) d = dot16<T>(qk[g][j], kr[r][j], d);
          d = group_sum<K::kC>(d);
          if (tok < n && (g % K::kC) == subk) s_buf[tok * GT + g] = d * a.scale_log2;
        }
      }
    }
    __syncthreads();

    // ---- softmax over the chunk: one wave per query row
    for (int g = w; g < GT; g += kWaves) {
      float mx = -INFINITY;
      for (int t = lane; t < n; t += kWave) mx = fmaxf(mx, s_buf[t * GT + g]);
      mx = wave_max(mx);
      const float m_old = s_m[g];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.0f;
      for (int t = lane; t < n; t += kWave) {
        const float e = __builtin_amdgcn_exp2f(s_buf[t * GT + g] - m_new);
        s_buf[t * GT + g] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        const float corr = __builtin_amdgcn_exp2f(m_old - m_new);  // 0 on the first chunk
        s_corr[g] = corr;
        s_l[g] = s_l[g] * corr + sum;
        s_m[g] = m_new;
      }
    }
    __syncthreads();

    // ---- V pass: acc = acc * corr + sum_t p_t v_t
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float corr = s_corr[g];
#pragma unroll
      for (int e = 0; e < K::kE; ++e) acc[g][e] *= corr;
    }
    for (int tile = w; tile * K::kTV < n; tile += kWaves) {
      u32x4 vr[K::kRV];
#pragma unroll
      for (int r = 0; r < K::kRV; ++r) {
        const int tok = tile * K::kTV + r * (kWave / K::kCV) + lane / K::kCV;
        int phys = (tok < n) ? s_tbl[tok >> a.log2_block] : 0;
        phys = phys < 0 ? 0 : phys;  // already flagged in the K pass
        vr[r] = load16(vbase + phys * block_stride + static_cast<int64_t>(tok & bmask) * D +
                       subv * K::kE);
      }
#pragma unroll
      for (int r = 0; r < K::kRV; ++r) {
        const int tok = tile * K::kTV + r * (kWave / K::kCV) + lane / K::kCV;
        if (tok < n) {  // rows past the chunk were read from block 0 and are never used
          float vf[K::kE];
          unpack16<T>(vr[r], vf);
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            const float p = s_buf[tok * GT + g];
#pragma unroll
            for (int e = 0; e < K::kE; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
          }
        }
      }
    }
  }

  // ---- combine: across the wave's token groups, then across waves in wave order
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < K::kE; ++e)
      for (int o = K::kCV; o < kWave; o <<= 1) acc[g][e] += __shfl_xor(acc[g][e], o);
  __syncthreads();  // probabilities are no longer needed
  if (lane < K::kCV) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int e = 0; e < K::kE; ++e) s_buf[(w * GT + g) * D + lane * K::kE + e] = acc[g][e];
  }
  __syncthreads();

  const bool bad = s_bad != 0;
  const float qnan = __builtin_nanf("");
  for (int i = tid; i < ng * D; i += kThreads) {
    const int g = i / D;
    const int d = i - g * D;
    float sum = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) sum += s_buf[(ww * GT + g) * D + d];
    const float l = s_l[g];
    const float o = bad ? qnan : sum / l;
    if (nparts == 1) {
      out[(row0 + g) * D + d] = static_cast<T>(o);
    } else {
      const int64_t idx = (row0 + g) * a.max_parts + part;
      a.ws_o[idx * D + d] = o;
      if (d == 0) {
        a.ws_m[idx] = bad ? qnan : s_m[g];
        a.ws_l[idx] = bad ? qnan : l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode, pass 2: merge the partitions of one (sequence, query head); thread d owns dim d
// ---------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(D) void pa_reduce_kernel(T* __restrict__ out,
                                                      const float* __restrict__ ws_m,
                                                      const float* __restrict__ ws_l,
                                                      const float* __restrict__ ws_o,
                                                      const int32_t* __restrict__ context_lens,
                                                      int num_q_heads, int max_context_len,
                                                      int partition_size, int max_parts) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const int ctx = context_lens[s];
  if (ctx <= 0 || ctx > max_context_len) return;  // pass 1 wrote zeros or NaN
  const int nparts = (ctx + partition_size - 1) / partition_size;
  if (nparts <= 1) return;  // pass 1 wrote the output directly
  const int64_t base = (static_cast<int64_t>(s) * num_q_heads + h) * max_parts;
  float big_m = -INFINITY;
  for (int p = 0; p < nparts; ++p) big_m = fmaxf(big_m, ws_m[base + p]);
  float num = 0.0f, den = 0.0f;
  for (int p = 0; p < nparts; ++p) {
    const float wgt = ws_l[base + p] * __builtin_amdgcn_exp2f(ws_m[base + p] - big_m);
    den += wgt;
    num = fmaf(wgt, ws_o[(base + p) * D + d], num);
  }
  out[(static_cast<int64_t>(s) * num_q_heads + h) * D + d] = static_cast<T>(num / den);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int log2_of(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int check_hip(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

int check_common(int dtype, int head_dim, int block_size) {
  if (dtype != PA_F32 && dtype != PA_F16) return fail(PA_ERR_UNSUPPORTED, "dtype %d is not PA_F32 or PA_F16", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d: only 8, 16 and 32 are built", block_size);
  return PA_OK;
}

struct DecodeGeom {
  int partition_size;  // effective (> 0)
  int max_parts;
  int gt;
  int n_gtiles;
  size_t ws_bytes;     // required workspace (0 when one partition covers every context)
};

int max_parts_for(int max_context_len, int partition_size) {
  if (max_context_len <= 0) return 1;
  return (max_context_len + partition_size - 1) / partition_size;
}

size_t workspace_for(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_parts) {
  const size_t per = static_cast<size_t>(num_seqs * num_q_heads * max_parts) * sizeof(float);
  return 2 * align256(per) + align256(per * static_cast<size_t>(head_dim));
}

struct DecodeCall {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale;
  int32_t block_size, num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
      max_context_len;
  int64_t num_blocks;
  int32_t partition_size, dtype;
  void* workspace;
  size_t workspace_bytes;
  hipStream_t stream;
};

int check_decode(const DecodeCall& c, DecodeGeom* g) {
  int rc = check_common(c.dtype, c.head_dim, c.block_size);
  if (rc != PA_OK) return rc;
  if (c.num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", c.num_seqs);
  if (c.num_kv_heads <= 0 || c.num_q_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d and num_kv_heads %d must be > 0", c.num_q_heads, c.num_kv_heads);
  if (c.num_q_heads % c.num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", c.num_q_heads, c.num_kv_heads);
  if (c.max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d must be > 0", c.max_blocks_per_seq);
  if (c.num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld must be > 0", (long long)c.num_blocks);
  if (c.max_context_len < 0) return fail(PA_ERR_INVALID_ARG, "max_context_len %d < 0", c.max_context_len);
  if (static_cast<int64_t>(c.max_context_len) > static_cast<int64_t>(c.max_blocks_per_seq) * c.block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len %d exceeds max_blocks_per_seq * block_size = %lld",
                c.max_context_len, (long long)c.max_blocks_per_seq * c.block_size);
  if (c.partition_size < 0 || c.partition_size % c.block_size != 0)
    return fail(PA_ERR_INVALID_ARG, "partition_size %d must be 0 or a positive multiple of block_size %d",
                c.partition_size, c.block_size);
  const int group = c.num_q_heads / c.num_kv_heads;
  g->gt = group >= 8 ? 8 : group >= 4 ? (group == 4 ? 4 : 8) : group >= 2 ? (group == 2 ? 2 : 4) : 1;
  g->n_gtiles = (group + g->gt - 1) / g->gt;
  if (static_cast<int64_t>(c.num_kv_heads) * g->n_gtiles > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d too large for one launch", c.num_q_heads);
  if (c.num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d > 65535", c.num_seqs);
  if (c.partition_size > 0) {
    g->partition_size = c.partition_size;
    g->max_parts = max_parts_for(c.max_context_len, c.partition_size);
  } else {
    // one partition per sequence: its length is the largest context, rounded to a whole chunk
    const int span = c.max_context_len > 0 ? c.max_context_len : 1;
    g->partition_size = (span + kChunk - 1) / kChunk * kChunk;
    g->max_parts = 1;
  }
  g->ws_bytes = g->max_parts > 1 ? workspace_for(c.num_seqs, c.num_q_heads, c.head_dim, g->max_parts) : 0;
  if (c.num_seqs == 0) return PA_OK;
  if (!c.out || !c.q || !c.k_cache || !c.v_cache || !c.block_tables || !c.context_lens)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(c.out, 16) || !aligned(c.q, 16) || !aligned(c.k_cache, 16) || !aligned(c.v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "out, q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(c.block_tables, 4) || !aligned(c.context_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables and context_lens must be 4-byte aligned");
  if (g->ws_bytes > 0) {
    if (!c.workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", g->ws_bytes);
    if (c.workspace_bytes < g->ws_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", c.workspace_bytes, g->ws_bytes);
    if (!aligned(c.workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  return PA_OK;
}

void split_workspace(const DecodeCall& c, const DecodeGeom& g, float** m, float** l, float** o) {
  if (g.ws_bytes == 0) {
    *m = *l = *o = nullptr;
    return;
  }
  const size_t per = static_cast<size_t>(c.num_seqs) * c.num_q_heads * g.max_parts * sizeof(float);
  char* base = static_cast<char*>(c.workspace);
  *m = reinterpret_cast<float*>(base);
  *l = reinterpret_cast<float*>(base + align256(per));
  *o = reinterpret_cast<float*>(base + 2 * align256(per));
}

template <typename T, int D, int GT>
int launch_partition(const DecodeCall& c, const DecodeGeom& g) {
  PartitionArgs a;
  a.out = c.out;
  split_workspace(c, g, &a.ws_m, &a.ws_l, &a.ws_o);
  a.q = c.q;
  a.k_cache = c.k_cache;
  a.v_cache = c.v_cache;
  a.block_tables = c.block_tables;
  a.context_lens = c.context_lens;
  a.scale_log2 = static_cast<float>(static_cast<double>(c.scale) * 1.4426950408889634);
  a.block_size = c.block_size;
  a.log2_block = log2_of(c.block_size);
  a.num_kv_heads = c.num_kv_heads;
  a.num_q_heads = c.num_q_heads;
  a.group = c.num_q_heads / c.num_kv_heads;
  a.n_gtiles = g.n_gtiles;
  a.max_blocks_per_seq = c.max_blocks_per_seq;
  a.max_context_len = c.max_context_len;
  a.num_blocks = c.num_blocks;
  a.partition_size = g.partition_size;
  a.max_parts = g.max_parts;
  const dim3 grid(g.max_parts, c.num_kv_heads * g.n_gtiles, c.num_seqs);
  hipLaunchKernelGGL((pa_partition_kernel<T, D, GT>), grid, dim3(kThreads), 0, c.stream, a);
  return check_hip("pa_partition_kernel launch");
}

template <typename T, int D>
int launch_partition_gt(const DecodeCall& c, const DecodeGeom& g) {
  switch (g.gt) {
    case 1: return launch_partition<T, D, 1>(c, g);
    case 2: return launch_partition<T, D, 2>(c, g);
    case 4: return launch_partition<T, D, 4>(c, g);
    default: return launch_partition<T, D, 8>(c, g);
  }
}

int run_partitions(const DecodeCall& c, const DecodeGeom& g) {
  if (c.num_seqs == 0) return PA_OK;
  if (c.dtype == PA_F16)
    return c.head_dim == 64 ? launch_partition_gt<f16, 64>(c, g) : launch_partition_gt<f16, 128>(c, g);
  return c.head_dim == 64 ? launch_partition_gt<float, 64>(c, g) : launch_partition_gt<float, 128>(c, g);
}

template <typename T, int D>
int launch_reduce(void* out, const float* m, const float* l, const float* o, const int32_t* ctx,
                  int num_seqs, int num_q_heads, int max_context_len, int partition_size,
                  int max_parts, hipStream_t stream) {
  const dim3 grid(num_q_heads, num_seqs);
  hipLaunchKernelGGL((pa_reduce_kernel<T, D>), grid, dim3(D), 0, stream, static_cast<T*>(out), m,
                     l, o, ctx, num_q_heads, max_context_len, partition_size, max_parts);
  return check_hip("pa_reduce_kernel launch");
}

int run_reduce(void* out, const int32_t* ctx, int num_seqs, int num_q_heads, int head_dim,
               int max_context_len, int dtype, const DecodeGeom& g, const void* workspace,
               hipStream_t stream) {
  if (num_seqs == 0 || g.max_parts <= 1) return PA_OK;
  const size_t per = static_cast<size_t>(num_seqs) * num_q_heads * g.max_parts * sizeof(float);
  const char* base = static_cast<const char*>(workspace);
  const float* m = reinterpret_cast<const float*>(base);
  const float* l = reinterpret_cast<const float*>(base + align256(per));
  const float* o = reinterpret_cast<const float*>(base + 2 * align256(per));
  if (dtype == PA_F16)
    return head_dim == 64 ? launch_reduce<f16, 64>(out, m, l, o, ctx, num_seqs, num_q_heads, max_context_len, g.partition_size, g.max_parts, stream)
                          : launch_reduce<f16, 128>(out, m, l, o, ctx, num_seqs, num_q_heads, max_context_len, g.partition_size, g.max_parts, stream);
  return head_dim == 64 ? launch_reduce<float, 64>(out, m, l, o, ctx, num_seqs, num_q_heads, max_context_len, g.partition_size, g.max_parts, stream)
                        : launch_reduce<float, 128>(out, m, l, o, ctx, num_seqs, num_q_heads, max_context_len, g.partition_size, g.max_parts, stream);
}

template <typename T, int D>
int launch_cache_write(const void* k, const void* v, const int64_t* slots, void* kc, void* vc,
                       int num_tokens, int num_kv_heads, int block_size, int64_t num_blocks,
                       hipStream_t stream) {
  constexpr int kChunksPerRow = D * static_cast<int>(sizeof(T)) / 16;
  const int64_t chunks = static_cast<int64_t>(num_tokens) * num_kv_heads * kChunksPerRow;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL((pa_cache_write_kernel<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const T*>(k), static_cast<const T*>(v), slots,
                     static_cast<T*>(kc), static_cast<T*>(vc), chunks, num_kv_heads, block_size,
                     num_blocks * block_size);
  return check_hip("pa_cache_write_kernel launch");
}

DecodeCall make_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                     int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                     int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                     int32_t max_context_len, int64_t num_blocks, int32_t partition_size,
                     int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  DecodeCall c;
  c.out = out;
  c.q = q;
  c.k_cache = k_cache;
  c.v_cache = v_cache;
  c.block_tables = block_tables;
  c.context_lens = context_lens;
  c.scale = scale;
  c.block_size = block_size;
  c.num_kv_heads = num_kv_heads;
  c.num_seqs = num_seqs;
  c.num_q_heads = num_q_heads;
  c.head_dim = head_dim;
  c.max_blocks_per_seq = max_blocks_per_seq;
  c.max_context_len = max_context_len;
  c.num_blocks = num_blocks;
  c.partition_size = partition_size;
  c.dtype = dtype;
  c.workspace = workspace;
  c.workspace_bytes = workspace_bytes;
  c.stream = static_cast<hipStream_t>(stream);
  return c;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

const char* pa_last_error(void) { return g_error.c_str(); }

int pa_abi_version(void) { return PA_ABI_VERSION; }

int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream) {
  g_error.clear();
  int rc = check_common(dtype, head_dim, block_size);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d must be > 0", num_kv_heads);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld must be > 0", (long long)num_blocks);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "k, v, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(PA_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PA_F16)
    return head_dim == 64 ? launch_cache_write<f16, 64>(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, block_size, num_blocks, st)
                          : launch_cache_write<f16, 128>(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, block_size, num_blocks, st);
  return head_dim == 64 ? launch_cache_write<float, 64>(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, block_size, num_blocks, st)
                        : launch_cache_write<float, 128>(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, block_size, num_blocks, st);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0 || partition_size <= 0)
    return 0;
  const int max_parts = max_parts_for(max_context_len, partition_size);
  if (max_parts <= 1) return 0;
  return workspace_for(num_seqs, num_q_heads, head_dim, max_parts);
}

int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                         int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int64_t num_blocks, int32_t partition_size,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_error.clear();
  const DecodeCall c = make_call(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                 block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                                 max_blocks_per_seq, max_context_len, num_blocks, partition_size,
                                 dtype, workspace, workspace_bytes, stream);
  DecodeGeom g;
  const int rc = check_decode(c, &g);
  if (rc != PA_OK) return rc;
  return run_partitions(c, g);
}

int pa_decode_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                     int32_t partition_size, int32_t dtype, const void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_error.clear();
  if (dtype != PA_F32 && dtype != PA_F16) return fail(PA_ERR_UNSUPPORTED, "dtype %d is not PA_F32 or PA_F16", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", head_dim);
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || partition_size < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size");
  if (num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d > 65535", num_seqs);
  if (partition_size == 0 || num_seqs == 0) return PA_OK;
  DecodeGeom g;
  g.partition_size = partition_size;
  g.max_parts = max_parts_for(max_context_len, partition_size);
  g.ws_bytes = g.max_parts > 1 ? workspace_for(num_seqs, num_q_heads, head_dim, g.max_parts) : 0;
  if (g.ws_bytes == 0) return PA_OK;
  if (!out || !context_lens) return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(out, 16) || !aligned(context_lens, 4)) return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", g.ws_bytes);
  if (workspace_bytes < g.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, g.ws_bytes);
  if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return run_reduce(out, context_lens, num_seqs, num_q_heads, head_dim, max_context_len, dtype, g,
                    workspace, static_cast<hipStream_t>(stream));
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
              int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
              int64_t num_blocks, int32_t partition_size, int32_t dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  g_error.clear();
  const DecodeCall c = make_call(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                 block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                                 max_blocks_per_seq, max_context_len, num_blocks, partition_size,
                                 dtype, workspace, workspace_bytes, stream);
  DecodeGeom g;
  int rc = check_decode(c, &g);
  if (rc != PA_OK) return rc;
  rc = run_partitions(c, g);
  if (rc != PA_OK) return rc;
  return run_reduce(out, context_lens, num_seqs, num_q_heads, head_dim, max_context_len, dtype, g,
                    workspace, c.stream);
}

}  // extern "C"
