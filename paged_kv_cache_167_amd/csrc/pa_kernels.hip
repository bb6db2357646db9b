// Paged KV-cache decode attention for MI355X (gfx950, CDNA4, wave64).
//
// Three kernels:
//   pa_cache_write_kernel  -- scatter each new token's K/V row into its slot.
//   pa_stream_kernel       -- attention over the paged K/V, the whole batch streamed
//                             by persistent waves that each own a share of it (equal
//                             in tiles plus piece boundaries, weighted by die).
//   pa_reduce_kernel       -- log-sum-exp merge of the pieces a context was split into.
//
// Sources (page title, section):
//  [DRV]  "揭开 NVIDIA 驱动栈的面纱：GPU 显存页表与 vLLM 中的 PagedAttention 是如何在底层协同的"
//         (kwkd.cn), section 6: block table lookup of a logical position and the
//         block * block-stride + head * head-stride + offset address of a K row.
//  [SRC]  vLLM source walk-through (peacm.com), section 3.2 (append into the last
//         block), section 3.4 (loop over logical blocks, tail mask, online softmax).
//  [CON]  "PagedAttention：当 KV Cache 遇到操作系统分页" (forceinjection.github.io),
//         section 3.2 (the kernel walks the table block by block); section 5.1 (the
//         software translation costs kernel time; keep the table lookups cheap).
//  [SOSP] "《Efficient Memory Management for LLM Serving with PagedAttention》深度解读报告"
//         (zako-mio.github.io), sections 2.3 and 3.3 (only the filled slots of a block
//         take part; the result equals attention over contiguous K/V).
//
// Design for gfx950 (not a translation of the pages' CUDA kernel):
//  * The pool layout [N, Hkv, B, D] makes one (block, kv head) tile a contiguous
//    B*D run; a wave reads 16 token rows at a time with 16-byte loads.
//  * All G query heads that share a kv head are handled by one wave, so each K/V
//    row is read from HBM once per group (GQA), not once per query head.
//  * Work split ("stream-K"): the batch is flattened into tiles of consecutive tokens
//    ordered by (sequence, kv head, position) and every persistent wave takes a
//    contiguous run of them, the runs equal in tiles plus one tile's worth per segment
//    they enter.  A context split between waves leaves one partial result per piece;
//    the reduce kernel merges the pieces by log-sum-exp.
//    Load balance is exact whatever the mix of context lengths.
//  * Each wave keeps a two-stage ring in LDS filled by direct global->LDS loads, so
//    two tiles are in flight during arithmetic without holding them in registers.
//    Block-table entries and context lengths are wave-uniform and come in through
//    scalar loads, which never wait behind the vector loads.
//  * C lanes share a token row for both K and V.  Scores: v_dot2 products of the
//    lane's 16-byte chunks with the matching q chunks, summed over the C lanes with
//    DPP row permutations fused into the adds; the probability is applied to the V
//    chunks the same lanes hold.  Each token group keeps its own online-softmax
//    state (running max and sum, [SRC] 3.4); the groups merge at the end of a piece.
//  * Results depend only on logical positions and the fixed work split, so they are
//    bitwise reproducible under any physical block placement or block size.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>

#include "pa.h"
#include "pa_internal.h"

namespace {

using f16 = _Float16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxWaves = 4096;  // persistent fp32 waves in the default split
constexpr int kMfWavesPerCU = 4;  // persistent fp16 waves per compute unit in the default split
constexpr int kMfStages = 3;      // LDS ring depth of the fp16 kernel
constexpr int kF8WavesPerCU = 8;  // E4M3 pools: tiles carry half the bytes, so more waves
constexpr int kF8Stages = 2;      // with a shallower ring keep more loads in flight per CU
// One-wave work-groups go to the eight dies in turn, so wave w runs on die w mod 8.  The
// odd-numbered dies of MI355X stream K/V 4-8 % slower than the even ones (measured per die on
// several boards), so the stream kernels give an odd-numbered wave a share of this weight
// (of 64) against an even one's -- on a whole device (all kWholeDeviceCUs compute units, eight
// dies); a partitioned one keeps equal weights.
constexpr int kOddDieWeight = 60;
constexpr int kWholeDeviceCUs = 256;

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float as_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned as_u(float f) { return __builtin_bit_cast(unsigned, f); }

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

// Wave-wide scans and reductions in registers: DPP row operations within each row of 16
// lanes, then across rows (row broadcasts for the scan, the permlane swaps, which pair lanes
// i, i ^ 32 and i, i ^ 16, for reductions).  Shuffles would take an LDS round trip per step.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_or_zero(int x) {  // lanes with no source, or outside ROWS: 0
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u(unsigned x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}

// op over all 64 lanes, result in every lane; op on the 32-bit patterns (as unsigned)
template <typename F>
__device__ __forceinline__ unsigned wave_all(unsigned x, F op) {
  x = op(x, dpp_u<0xB1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_u<0x4E>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_u<0x141>(x));  // row_half_mirror
  x = op(x, dpp_u<0x140>(x));  // row_mirror: the row's result in all its lanes
  const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return op(b[0], b[1]);
}

__device__ __forceinline__ int wave_sum_int(int x) {
  const unsigned r = wave_all(static_cast<unsigned>(x), [](unsigned u, unsigned v) { return u + v; });
  return __builtin_amdgcn_readfirstlane(static_cast<int>(r));
}

// inclusive prefix sum over the lanes
__device__ __forceinline__ int wave_incl_scan_int(int x) {
  x += dpp_or_zero<0x111, 0xF>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xF>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xF>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xF>(x);  // row_shr:8: the scan within each row
  x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15: rows 1 and 3 add the row before
  x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31: rows 2 and 3 add rows 0-1
  return x;
}

__device__ __forceinline__ int wave_min_int(int x) {
  const unsigned r = wave_all(static_cast<unsigned>(x), [](unsigned u, unsigned v) {
    return static_cast<unsigned>(min(static_cast<int>(u), static_cast<int>(v)));
  });
  return __builtin_amdgcn_readfirstlane(static_cast<int>(r));
}

__device__ __forceinline__ float wave_max(float x) {
  return __builtin_bit_cast(float, wave_all(__builtin_bit_cast(unsigned, x), [](unsigned u, unsigned v) {
    return __builtin_bit_cast(unsigned, fmaxf(__builtin_bit_cast(float, u), __builtin_bit_cast(float, v)));
  }));
}

__device__ __forceinline__ float wave_sum(float x) {
  return __builtin_bit_cast(float, wave_all(__builtin_bit_cast(unsigned, x), [](unsigned u, unsigned v) {
    return __builtin_bit_cast(unsigned, __builtin_bit_cast(float, u) + __builtin_bit_cast(float, v));
  }));
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

// acc[j*E + e] += p * v[j][e] over the lane's chunks of one V row (fp16 halves go
// straight into v_fma_mix_f32).
template <typename T>
struct PV;

template <>
struct PV<f16> {
  template <int NL>
  __device__ __forceinline__ static void run(float* acc, float p, const u32x4 (&v)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x2 h = word_as<f16x2>(v[j], i);
        acc[j * 8 + 2 * i] = fmaf(p, static_cast<float>(h.x), acc[j * 8 + 2 * i]);
        acc[j * 8 + 2 * i + 1] = fmaf(p, static_cast<float>(h.y), acc[j * 8 + 2 * i + 1]);
      }
  }
};

template <>
struct PV<float> {
  template <int NL>
  __device__ __forceinline__ static void run(float* acc, float p, const u32x4 (&v)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j * 4 + i] = fmaf(p, word_as<float>(v[j], i), acc[j * 4 + i]);
  }
};

// Pack E fp32 values into one 16-byte chunk of T (round to nearest even for fp16).
template <typename T>
__device__ __forceinline__ u32x4 pack16(const float* x);

template <>
__device__ __forceinline__ u32x4 pack16<f16>(const float* x) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = {static_cast<f16>(x[2 * i]), static_cast<f16>(x[2 * i + 1])};
    r[i] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

template <>
__device__ __forceinline__ u32x4 pack16<float>(const float* x) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, x[i]);
  return r;
}

// 2^(a - b) that is 0 when a is -inf (an empty running state), never NaN.
__device__ __forceinline__ float rescale(float a, float b) {
  return a == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(a - b);
}

// A wave-uniform 32-bit load through the scalar unit (the address is in SGPRs).  Its
// completion is tracked by lgkmcnt, so waiting for it never waits for the K/V loads in
// flight.  Written as asm because the compiler emits a vector load (and a wait for every
// outstanding vector load) wherever it cannot prove the memory unmodified since entry.
__device__ __forceinline__ int32_t scalar_load(const int32_t* p) {
  // readfirstlane keeps the address in SGPRs even where the compiler computed it in VGPRs
  const uint64_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int32_t* q = reinterpret_cast<const int32_t*>((static_cast<uint64_t>(hi) << 32) | lo);
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q));
  return v;
}

// Read one ring stage back: wait until at most VMCNT vector-memory operations are
// outstanding (the stage's own direct-to-LDS loads are older than those, and loads
// complete in order), then read the lane's eight 16-byte words at base + 16*lane +
// 1024*i, then wait for the reads.  Written as one asm block so that the compiler's
// conservative tracking of direct-to-LDS loads cannot add a full drain in front of the
// reads; the memory clobber keeps every other memory access on its side of the block.
template <int VMCNT>
__device__ __forceinline__ void read_stage8(uint32_t lds_addr, u32x4 (&o)[8]) {
  asm volatile(
      "s_waitcnt vmcnt(%9)\n\t"
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(o[0]), "=v"(o[1]), "=v"(o[2]), "=v"(o[3]), "=v"(o[4]), "=v"(o[5]), "=v"(o[6]),
        "=v"(o[7])
      : "v"(lds_addr), "n"(VMCNT)
      : "memory");
}

// Lanes that share one token row.  Each lane keeps its q chunks in registers, so the
// row is split finely enough that they stay near 32 VGPRs.  At least 8 lanes per row:
// a row slot then spans at most 64/8 = 8 consecutive tokens, which never straddle a
// block (B >= 8), so its block-table entry is one wave-uniform scalar load.  At most
// 16 lanes (one DPP row) and at most the row's number of 16-byte chunks.
constexpr int pick_row_lanes(int row_bytes, int gt) {
  const int cv = row_bytes / 16;
  int c = gt * row_bytes / 128;
  if (c < 8) c = 8;
  if (c > 16) c = 16;
  if (c > cv) c = cv;
  return c;
}

template <typename T, int D, int GT>
struct Cfg {
  static constexpr int kRow = D * static_cast<int>(sizeof(T));  // bytes per token row
  static constexpr int kE = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
  static constexpr int kCV = kRow / 16;                         // 16-byte chunks per row
  static constexpr int kC = pick_row_lanes(kRow, GT);           // lanes per token row
  static constexpr int kNL = kCV / kC;                          // chunks per lane per row
  static constexpr int kDL = kNL * kE;                          // elements per lane per row
  static constexpr int kGroups = kWave / kC;                    // token groups in a wave
  static constexpr int kRK = 4 / kNL;                           // rows per lane per tile
  static constexpr int kTK = kRK * kGroups;                     // tokens per tile
  static constexpr int kSlots = kRK * kNL * 2;                  // 1 KB LDS slots per tile
  static_assert(kC * kNL == kCV && kNL <= 4, "row split");
  static_assert(kSlots == 8, "a tile is eight 1 KB slots (read_stage8)");
  static_assert(kGroups <= 8, "a row slot must lie in one block of at least 8 tokens");
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
  // the row loads do not wait for the slot: all three are in flight together
  const int64_t src = row * D + c * kE;
  const u32x4 kx = load16(k + src);
  const u32x4 vx = load16(v + src);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * D + c * kE;
  *reinterpret_cast<u32x4*>(k_cache + dst) = kx;
  *reinterpret_cast<u32x4*>(v_cache + dst) = vx;
}

// An E4M3 store scale: the scale s (positive, finite) and 1/s rounded once to fp32.
struct F8Scale {
  float s, inv;
};

// E4M3 code nearest to the exact quotient x / s (ties to the even code), saturated to +-448;
// +-0 stays +-0 and any NaN becomes 0x7F (its sign carries no value).  The value of the code
// goes to `val` (every E4M3 value is exact in fp16).
// y = x * inv lies within about 2^-22 of x / s (relative).  Rounding |y| toward zero onto
// the E4M3 grid gives a code c0 such that |x| / s rounds to c0 or to c0 + 1 (the next value
// up): where |y| and |x| / s fall on two sides of a code value, that value is the nearest to
// both.  The midpoint m between the two values decides, by the sign of |x| - m s, which one
// fma gives with a single rounding: it is zero only when |x| / s equals m (then the even
// code), and otherwise far above the fp32 subnormal range.  Normal range: truncate the fp32
// bit pattern to 3 mantissa bits and rebase the exponent from bias 127 to 7 (the midpoint
// sets the fourth mantissa bit).  Below 2^-6 the codes are steps of 2^-9.
__device__ __forceinline__ uint32_t e4m3_code_exact(float x, F8Scale sc, float& val) {
  const float ax = __builtin_fabsf(x);
  const float a = __builtin_fabsf(x * sc.inv);
  const uint32_t mag = as_u(a);
  const bool nrm = a >= 0.015625f;
  const float k = __builtin_fminf(__builtin_floorf(a * 512.0f), 7.0f);  // below 2^-6: 0..7; NaN: 7
  const uint32_t c0 = nrm ? (mag >> 20) - (120u << 3) : static_cast<uint32_t>(k);
  const float v0 = nrm ? as_f(mag & 0xFFF00000u) : k * (1.0f / 512.0f);
  const float m = nrm ? as_f((mag & 0xFFF00000u) | 0x00080000u) : (k + 0.5f) * (1.0f / 512.0f);
  const float r = __builtin_fmaf(-m, sc.s, ax);
  const bool up = r > 0.0f || (r == 0.0f && (c0 & 1u) != 0u);
  uint32_t c = up ? c0 + 1u : c0;
  float v = up ? 2.0f * m - v0 : v0;  // the next value up, exactly
  const bool sat = a >= 448.0f;       // infinities too
  c = sat ? 0x7Eu : c;
  v = sat ? 448.0f : v;
  const bool zero = ax == 0.0f;  // also when inv overflowed to infinity (x * inv is NaN)
  c = zero ? 0u : c;
  v = zero ? 0.0f : v;
  const bool nan = !(ax == ax);
  val = nan ? __builtin_nanf("") : as_f(as_u(v) | (as_u(x) & 0x80000000u));
  return nan ? 0x7Fu : (c | ((as_u(x) >> 24) & 0x80u));
}

// Eight fp16 values stored with scale sc, as eight E4M3 codes (byte i = element i).
__device__ __forceinline__ u32x2 encode8(const u32x4& x, F8Scale sc) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f16x2 h = word_as<f16x2>(x, i / 2);
    float val;
    w[i / 4] |= e4m3_code_exact(static_cast<float>(h[i % 2]), sc, val) << (8 * (i % 4));
  }
  return u32x2{w[0], w[1]};
}

// E4M3 pools: one thread per 16 codes (two 16-byte fp16 chunks) of one (token, kv head)
// row.  Each element is stored as the code nearest to x / scale.
template <int D>
__global__ __launch_bounds__(256) void pa_cache_write_fp8_kernel(
    const f16* __restrict__ k, const f16* __restrict__ v, const int64_t* __restrict__ slot_mapping,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, F8Scale ks, F8Scale vs,
    int64_t num_chunks, int num_kv_heads, int block_size, int64_t num_slots) {
  constexpr int kChunksPerRow = D / 16;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= num_chunks) return;
  const int c = static_cast<int>(i % kChunksPerRow);
  const int64_t row = i / kChunksPerRow;  // = t * Hkv + h
  const int h = static_cast<int>(row % num_kv_heads);
  const int64_t t = row / num_kv_heads;
  const int64_t src = row * D + c * 16;
  const u32x4 k0 = load16(k + src), k1 = load16(k + src + 8);
  const u32x4 v0 = load16(v + src), v1 = load16(v + src + 8);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * D + c * 16;
  const u32x2 ka = encode8(k0, ks), kb = encode8(k1, ks);
  const u32x2 va = encode8(v0, vs), vb = encode8(v1, vs);
  *reinterpret_cast<u32x4*>(k_cache + dst) = u32x4{ka[0], ka[1], kb[0], kb[1]};
  *reinterpret_cast<u32x4*>(v_cache + dst) = u32x4{va[0], va[1], vb[0], vb[1]};
}

// ---------------------------------------------------------------------------
// decode, pass 1: persistent waves streaming equal shares of the batch
// ---------------------------------------------------------------------------

// A segment is one (sequence, unit) pair, unit = (kv head, tile of GT query heads);
// it has ceil(ctx / TK) tiles.  Segments are ordered by sequence, then unit.
struct StreamArgs {
  void* out;
  int2* seg_desc;       // [S * n_units] {first wave, last wave} holding pieces of the segment, or
                        // with partitions {first partition record, partitions}
  float* rec_m;         // [records * rec_rows] per piece record: running max (log2 units) per row
  float* rec_l;         // [records * rec_rows] exp-sum per row
  float* rec_o;         // [records * rec_rows * D] normalised output per row
  int part_tiles;       // > 0: pieces are fixed partitions of this many tiles (one record each)
  int odd_weight;       // share weight (of 64) of an odd-numbered wave: kOddDieWeight or 64
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
  int group;     // query heads per kv head
  int n_gtiles;  // ceil(group / GT)
  int n_units;   // num_kv_heads * n_gtiles
  int num_seqs;
  int max_blocks_per_seq;
  int max_context_len;
  int64_t num_blocks;
  int num_waves;
  int rec_rows;     // query rows per piece record
  float out_scale;  // E4M3 pools: the V scale, applied to the normalised output
  // virtually contiguous cache (no table): sequence s's token p of kv head h is at
  // dense_k + s * seq_bytes + p * token_bytes + h * row bytes; phantom tiles read guard_k
  const char* dense_k;
  const char* dense_v;
  const char* guard_k;
  const char* guard_v;
  int64_t seq_bytes;
  int64_t token_bytes;
  // append mode: the token at position ctx - 1 of sequence s is read from these rows
  // ([num_seqs, num_kv_heads, head_dim]) instead of the pools
  const char* k_new;
  const char* v_new;
  F8Scale k_sc, v_sc;  // E4M3 append mode: the scales the new rows are coded with
};

// Append mode of the reduce kernel: where the new tokens' rows go (k_new == nullptr: off).
struct AppendArgs {
  const char* k_new;  // [num_seqs, num_kv_heads, head_dim] rows of the pools' element type, or
  const char* v_new;  // fp16 rows for E4M3 pools
  char* k_cache;      // the pools
  char* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  int block_size;
  int num_kv_heads;
  int64_t num_blocks;
  int codes;           // E4M3 pools: store the code nearest to x / scale of each element
  F8Scale k_sc, v_sc;
};

// Position of a wave in the flattened tile list (all wave-uniform, in SGPRs).
struct Cursor {
  int s;       // sequence
  int unit;    // kv head * n_gtiles + query-head tile
  int t;       // tile within the segment
  int nt;      // tiles in the segment
  int ctx;     // context length of the sequence
  int gstart;  // global index of the segment's first tile
  int seg;     // non-empty segments before this one
  int p0;      // with partitions: the record of the segment's first partition
};

// The work split.  The batch is one list of tiles (TK consecutive tokens of one segment,
// segments in order), and each wave takes a share of an estimated cost: a tile costs one
// unit, and each piece boundary one more (a boundary -- q rows, record, cursor -- costs
// about as much as a tile on MI355X), so that a wave whose share crosses more boundaries
// takes fewer tiles.  The shares are weighted by die: wave w takes the positions
// [th(w), th(w + 1)), th(v) = ceil(cum_weight(v) total / Om), an odd-numbered wave weighing
// kOddDieWeight / 64 of an even one (equal weights for batches under two positions a wave).
//  * Default (part_tiles = 0): a boundary per non-empty segment.  Tile x of a segment with j
//    non-empty segments before it sits at cost position x + j + 1, and a share is a
//    contiguous range of tiles.  Wp = min(waves, total): every share is at least one
//    position wide, so every wave in a segment's {first, last} range holds a piece of it, as
//    the reduce requires.
//  * Partitions (part_tiles = PT > 0): each segment is cut into partitions of PT tiles (the
//    last may be shorter), a boundary each, and whole partitions go to the waves: partition
//    k, with first tile x and k partitions before it, sits at x + k + 1, and goes to the
//    wave whose share holds that position.  A partition is one piece with a record of its
//    own, so a sequence's result does not depend on the rest of the batch or on the wave
//    count.
template <int TK>
struct Work {
  const int32_t* ctxs;
  int S, max_ctx, n_units;
  int PT;           // tiles per partition, 0: none
  int Wp;           // waves sharing the work
  int total;        // tiles plus pieces (the host bounds it below 2^31)
  double inv_total;
  int wo;           // share weight (of 64) of an odd-numbered wave
  int64_t Om;       // total weight of the Wp waves
  double inv_om;
  int A, n_my;      // this wave's share: tiles [A, A + n_my)
  int ctx0;         // this lane's context length among the first 64 sequences (0 past S): one
                    // load serves the totals and the scan

  __device__ int seg_tiles(int ctx) const {  // invalid or empty contexts contribute no tiles
    return (ctx > 0 && ctx <= max_ctx) ? (ctx + TK - 1) / TK : 0;
  }
  __device__ int parts_of(int nt) const { return PT > 0 ? (nt + PT - 1) / PT : (nt > 0 ? 1 : 0); }
  // pieces start and end at segment ends, and with partitions at partition ends
  __device__ bool piece_starts(const Cursor& c) const { return c.t == 0 || (PT > 0 && c.t % PT == 0); }
  __device__ bool piece_ends(const Cursor& c) const {
    return c.t == c.nt - 1 || (PT > 0 && (c.t + 1) % PT == 0);
  }
  __device__ int part_record(const Cursor& c) const { return c.p0 + c.t / PT; }
  // summed share weights of waves 0 .. v - 1
  __device__ int64_t cum_weight(int v) const {
    return 64 * static_cast<int64_t>((v + 1) / 2) + static_cast<int64_t>(wo) * (v / 2);
  }

  // floor(n / d) for 0 <= n < 2^53 and 0 < d < 2^31: a double estimate (off by at most one
  // for these sizes), corrected with exact integer products
  __device__ static int64_t div_floor(int64_t n, int64_t d, double inv_d) {
    int64_t q = static_cast<int64_t>(static_cast<double>(n) * inv_d);
    if (q * d > n) --q;
    else if ((q + 1) * d <= n) ++q;
    return q;
  }

  // Split the work and place cursor c at this wave's first tile (n_my = 0: nothing to do).
  __device__ void init(const StreamArgs& a, int w, int lane, Cursor& c) {
    ctxs = a.context_lens;
    S = a.num_seqs;
    max_ctx = a.max_context_len;
    n_units = a.n_units;
    PT = a.part_tiles;
    n_my = 0;
    A = 0;
    ctx0 = lane < S ? ctxs[lane] : 0;
    int part = seg_tiles(ctx0), npc = parts_of(part);
    for (int b = kWave; b < S; b += kWave) {
      const int nt = (b + lane < S) ? seg_tiles(ctxs[b + lane]) : 0;
      part += nt;
      npc += parts_of(nt);
    }
    const int T = wave_sum_int(part) * n_units;
    total = T + wave_sum_int(npc) * n_units;
    Wp = min(a.num_waves, total);
    if (T == 0 || w >= Wp) return;
    inv_total = 1.0 / static_cast<double>(total);
    // wave w takes positions [th(w), th(w + 1)), th(v) = ceil(cum_weight(v) total / Om).  With
    // total >= 2 Wp every share is at least one position wide (an odd wave's is at least
    // floor(2 wo / 64) >= 1), so every wave in a segment's {first, last} range holds a piece
    // of it; smaller batches take equal weights.
    wo = total >= 2 * Wp ? a.odd_weight : 64;
    Om = cum_weight(Wp);
    inv_om = 1.0 / static_cast<double>(Om);
    const int th0 = static_cast<int>(div_floor(cum_weight(w) * total + Om - 1, Om, inv_om));
    const int th1 = w + 1 == Wp ? total : static_cast<int>(div_floor(cum_weight(w + 1) * total + Om - 1, Om, inv_om));
    // the first tiles at positions >= th0 and >= th1 (th1 = total: none, the end); with
    // partitions, the first tiles of the first partitions there
    int x0 = -1, x1 = T;
    int base_t = 0, base_j = 0;  // tiles and pieces (segments, or partitions) before the chunk
    for (int b = 0; b < S && x1 == T; b += kWave) {
      const int cl = b == 0 ? ctx0 : ((b + lane < S) ? ctxs[b + lane] : 0);
      const int nt = seg_tiles(cl), np = parts_of(nt);
      const int ts = nt * n_units, ss = np * n_units;
      const int ti = wave_incl_scan_int(ts), si = wave_incl_scan_int(ss);
      const int Gs = base_t + ti - ts, Js = base_j + si - ss;
      // the position of the sequence's last piece (the last tile of its last segment, or
      // the first tile of its last partition); the first sequence whose last reaches th
      // holds the first tile or partition at or past th
      const int last = PT > 0 ? Gs + Js + (n_units - 1) * (nt + np) + (np - 1) * (PT + 1) + 1 : Gs + ts + Js + ss - 1;
      auto find = [&](int th, int& x, bool cursor) __attribute__((always_inline)) {
        const uint64_t hit = __builtin_amdgcn_ballot_w64(nt > 0 && last >= th);
        if (hit == 0) return;
        const int l = __builtin_ctzll(hit);
        const int ntl = __builtin_amdgcn_readlane(nt, l), npl = __builtin_amdgcn_readlane(np, l);
        const int Gl = __builtin_amdgcn_readlane(Gs, l), Jl = __builtin_amdgcn_readlane(Js, l);
        const int gj = Gl + Jl;
        int u, t;
        if (PT > 0) {
          // partition j of unit u sits at gj + u (nt + np) + j (PT + 1) + 1
          const int ru = th - gj - (npl - 1) * (PT + 1) - 1;
          u = ru > 0 ? (ru + ntl + npl - 1) / (ntl + npl) : 0;
          const int rj = th - gj - u * (ntl + npl) - 1;
          t = (rj > 0 ? (rj + PT) / (PT + 1) : 0) * PT;
        } else {
          // unit u's last tile sits at gj + (u + 1)(nt + 1) - 1, its tile t at gj + u (nt + 1) + t + 1
          const int ru = th - gj + 1;
          u = ru > 0 ? max(0, (ru + ntl) / (ntl + 1) - 1) : 0;
          const int rt = th - gj - u * (ntl + 1) - 1;
          t = rt > 0 ? rt : 0;
        }
        x = Gl + u * ntl + t;
        if (cursor) {
          c.s = b + l;
          c.ctx = __builtin_amdgcn_readlane(cl, l);
          c.nt = ntl;
          c.unit = u;
          c.t = t;
          c.gstart = Gl + u * ntl;
          c.seg = Jl + u;            // default split: non-empty segments before
          c.p0 = Jl + u * npl;       // partitions: the segment's first partition
        }
      };
      if (x0 < 0) find(th0, x0, true);
      if (w + 1 < Wp) find(th1, x1, false);
      base_t += __builtin_amdgcn_readlane(ti, kWave - 1);
      base_j += __builtin_amdgcn_readlane(si, kWave - 1);
    }
    A = x0;
    n_my = x0 < 0 ? 0 : x1 - x0;
  }

  // the wave holding the last tile of c's segment (default split): the last wave v with
  // th(v) <= p, i.e. cum_weight(v) <= X = floor(p Om / total); waves 2k and 2k + 1 start at
  // weights k (64 + wo) and k (64 + wo) + 64
  __device__ int wave_of_last(const Cursor& c) const {
    const int p = c.gstart + c.nt - 1 + c.seg + 1;
    const int X = static_cast<int>(div_floor(static_cast<int64_t>(p) * Om, total, inv_total));
    const int k = X / (64 + wo);
    return min(2 * k + (X - k * (64 + wo) >= 64 ? 1 : 0), Wp - 1);
  }

  __device__ void advance(Cursor& c) const {
    if (++c.t < c.nt) return;
    c.gstart += c.nt;
    c.p0 += parts_of(c.nt);
    c.t = 0;
    ++c.seg;
    if (++c.unit < n_units) return;
    c.unit = 0;
    do {
      ++c.s;
      c.ctx = c.s < S ? scalar_load(ctxs + c.s) : 0;
      c.nt = seg_tiles(c.ctx);
    } while (c.nt == 0 && c.s < S);
  }
};

// ---------------------------------------------------------------------------
// merging the pieces of a split context (log-sum-exp over pieces, in token order)
// ---------------------------------------------------------------------------

// One wave merges query row g of a segment whose pieces are the records of waves
// first .. first + npieces - 1: the tail record of the first, then the head records of
// the others.  Piece p has running max m_p (log2 units), exp-sum l_p and normalised
// output o_p; with M = max m_p, out = sum_p w_p o_p / sum_p w_p, w_p = l_p 2^(m_p - M),
// accumulated in piece order.  Lane p holds piece p's (m, l); the weights are broadcast
// with readlane and each lane sums the outputs of its dims.
template <typename T, int D>
__device__ __forceinline__ void merge_row(T* dst, const float* rec_m, const float* rec_l,
                                          const float* rec_o, int first, int npieces, int rec_rows,
                                          int g, int lane) {
  constexpr int kDPL = D / kWave;  // dims per lane
  constexpr int kU = 4;            // piece outputs loaded together
  auto rec_of = [&](int p) { return p == 0 ? first * 2 + 1 : (first + p) * 2; };
  auto out_of = [&](int p) { return rec_o + (static_cast<int64_t>(rec_of(p)) * rec_rows + g) * D; };
  float big_m = -INFINITY, den = 0.0f;
  float num[kDPL];
#pragma unroll
  for (int k = 0; k < kDPL; ++k) num[k] = 0.0f;
  for (int p0 = 0; p0 < npieces; p0 += kWave) {
    const int p = p0 + lane;
    const int cnt = min(kWave, npieces - p0);
    const int r = p < npieces ? rec_of(p) * rec_rows + g : 0;
    const float mp = p < npieces ? rec_m[r] : -INFINITY;
    const float lp = p < npieces ? rec_l[r] : 0.0f;
    float ov[kU][kDPL];  // outputs of the first pieces, loaded alongside the maxima and sums
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int k = 0; k < kDPL; ++k) ov[u][k] = u < cnt ? out_of(p0 + u)[k * kWave + lane] : 0.0f;
    const float m_new = fmaxf(big_m, wave_max(mp));
    const float c_old = rescale(big_m, m_new);
    const float wp = p < npieces ? lp * __builtin_amdgcn_exp2f(mp - m_new) : 0.0f;
    den = den * c_old + wave_sum(wp);
#pragma unroll
    for (int k = 0; k < kDPL; ++k) num[k] *= c_old;
    for (int i = 0; i < cnt; i += kU) {
      if (i > 0) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int k = 0; k < kDPL; ++k) ov[u][k] = i + u < cnt ? out_of(p0 + i + u)[k * kWave + lane] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (i + u < cnt) {  // pieces in order
          const float wgt = as_f(__builtin_amdgcn_readlane(as_u(wp), i + u));
#pragma unroll
          for (int k = 0; k < kDPL; ++k) num[k] = fmaf(wgt, ov[u][k], num[k]);
        }
      }
    }
    big_m = m_new;
  }
#pragma unroll
  for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<T>(num[k] / den);
}

// The merge of merge_row over any list of pieces: piece p's running max, exp-sum and
// normalised output are record row idx(p) (record * rows per record + row), pieces in token
// order; the same arithmetic, in the same order.
template <typename T, int D, typename Idx>
__device__ __forceinline__ void merge_indexed(T* dst, const float* rec_m, const float* rec_l, const float* rec_o,
                                              int npieces, Idx idx, int lane) {
  constexpr int kDPL = D / kWave;
  constexpr int kU = 4;
  auto out_of = [&](int p) { return rec_o + static_cast<int64_t>(idx(p)) * D; };
  float big_m = -INFINITY, den = 0.0f;
  float num[kDPL];
#pragma unroll
  for (int k = 0; k < kDPL; ++k) num[k] = 0.0f;
  for (int p0 = 0; p0 < npieces; p0 += kWave) {
    const int p = p0 + lane;
    const int cnt = min(kWave, npieces - p0);
    const int r = p < npieces ? idx(p) : 0;
    const float mp = p < npieces ? rec_m[r] : -INFINITY;
    const float lp = p < npieces ? rec_l[r] : 0.0f;
    float ov[kU][kDPL];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int k = 0; k < kDPL; ++k) ov[u][k] = u < cnt ? out_of(p0 + u)[k * kWave + lane] : 0.0f;
    const float m_new = fmaxf(big_m, wave_max(mp));
    const float c_old = rescale(big_m, m_new);
    const float wp = p < npieces ? lp * __builtin_amdgcn_exp2f(mp - m_new) : 0.0f;
    den = den * c_old + wave_sum(wp);
#pragma unroll
    for (int k = 0; k < kDPL; ++k) num[k] *= c_old;
    for (int i = 0; i < cnt; i += kU) {
      if (i > 0) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int k = 0; k < kDPL; ++k) ov[u][k] = i + u < cnt ? out_of(p0 + i + u)[k * kWave + lane] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (i + u < cnt) {
          const float wgt = as_f(__builtin_amdgcn_readlane(as_u(wp), i + u));
#pragma unroll
          for (int k = 0; k < kDPL; ++k) num[k] = fmaf(wgt, ov[u][k], num[k]);
        }
      }
    }
    big_m = m_new;
  }
#pragma unroll
  for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<T>(num[k] / den);
}

template <typename T, int D, int GT>
__global__ __launch_bounds__(kWave) void pa_stream_kernel(const StreamArgs a) {
  using K = Cfg<T, D, GT>;
  constexpr int RK = K::kRK, NL = K::kNL, DL = K::kDL, C = K::kC, E = K::kE, TK = K::kTK;
  static_assert(16 % TK == 0, "partitions are whole multiples of 16 tokens: whole tiles");
  constexpr int GR = K::kGroups;
  __shared__ __align__(16) u32x4 s_stage0[8][kWave];
  __shared__ __align__(16) u32x4 s_stage1[8][kWave];

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int sub = lane % C;  // which chunks of a row this lane holds
  const int grp = lane / C;  // which token of a row slot this lane holds

  // ---- this wave's share of the batch's tiles, and the cursor at its first tile
  Work<TK> wk;
  Cursor cc;  // the tile being computed
  wk.init(a, w, lane, cc);
  const int n_my = wk.n_my;
  if (n_my == 0) return;
  const int A = wk.A, A_end = A + n_my;
  auto advance = [&](Cursor& c) { wk.advance(c); };

  // ---- direct-to-LDS loads of one tile into a ring stage
  const char* kcache = static_cast<const char*>(a.k_cache);
  const char* vcache = static_cast<const char*>(a.v_cache);
  const uint32_t head_bytes = static_cast<uint32_t>(a.block_size * D * sizeof(T));
  const uint32_t block_bytes = head_bytes * static_cast<uint32_t>(a.num_kv_heads);
  const int bmask = a.block_size - 1;
  // Issue the loads of tile f (a phantom tile past the wave's share reads rows of
  // block 0, kv head 0: a valid address whose data is never used).  Returns whether a
  // table entry of the tile lies outside the pool (then block 0 is read instead).
  auto fetch = [&](const Cursor& f, bool real, int st) -> bool {
    bool bad = false;
    const int kvh = real ? f.unit / a.n_gtiles : 0;
    const int32_t* trow = a.block_tables + static_cast<int64_t>(real ? f.s : 0) * a.max_blocks_per_seq;
    int p = 0, p_idx = -1;  // table entry of the previous row slot and its index
#pragma unroll
    for (int r = 0; r < RK; ++r) {
      const int tok0 = f.t * TK + r * GR;  // first token of the row slot (wave-uniform)
      const int idx = tok0 >> a.log2_block;
      if (!(real && tok0 < f.ctx)) {
        p = 0;
        p_idx = -1;
      } else if (idx != p_idx) {  // row slots of one block share the entry
        p = scalar_load(trow + idx);
        p_idx = idx;
        if (p < 0 || p >= a.num_blocks) {
          bad = true;
          p = 0;
        }
      }
      const uint32_t row = static_cast<uint32_t>(((tok0 + grp) & bmask) * D * sizeof(T)) +
                           static_cast<uint32_t>(sub * 16);
      const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(p)) * block_bytes +
                           static_cast<uint64_t>(kvh) * head_bytes + row;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        u32x4* slot = st == 0 ? &s_stage0[(r * NL + j) * 2][0] : &s_stage1[(r * NL + j) * 2][0];
        __builtin_amdgcn_global_load_lds(kcache + off + j * C * 16, slot, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vcache + off + j * C * 16, slot + kWave, 16, 0, 0);
      }
    }
    return bad;
  };
  const uint32_t stage_lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_stage0[0][lane]));
  const uint32_t stage_lds1 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_stage1[0][lane]));
  // Read a stage back (each lane reads the 16-byte words it loaded).  At least 8 loads
  // are issued after a stage's own loads before it is read, so waiting until at most 8
  // are outstanding never waits for less than that stage.
  auto unstage = [&](int st, u32x4 (&kb)[RK][NL], u32x4 (&vb)[RK][NL]) {
    u32x4 o[8];
    read_stage8<8>(st == 0 ? stage_lds0 : stage_lds1, o);
#pragma unroll
    for (int r = 0; r < RK; ++r)
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        kb[r][j] = o[(r * NL + j) * 2];
        vb[r][j] = o[(r * NL + j) * 2 + 1];
      }
  };

  // ---- per-piece state: q rows, and per token group the running max, sum, output
  u32x4 qv[GT][NL];
  float m[GT], l[GT], acc[GT][DL];
  int h0 = 0, ng = 0;
  bool piece_bad = false;
  const T* qp = static_cast<const T*>(a.q);

  auto piece_start = [&]() {
    const int kvh = cc.unit / a.n_gtiles;
    const int gtile = cc.unit - kvh * a.n_gtiles;
    h0 = kvh * a.group + gtile * GT;
    ng = min(GT, a.group - gtile * GT);
    const int64_t row0 = static_cast<int64_t>(cc.s) * a.num_q_heads + h0;
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int j = 0; j < NL; ++j)
        qv[g][j] = (g < ng) ? load16(qp + (row0 + g) * D + (j * C + sub) * E) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.0f;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[g][e] = 0.0f;
    }
    piece_bad = false;
    if (cc.t == 0 && lane == 0)  // this wave starts the segment: where its pieces are (waves, or partitions)
      a.seg_desc[cc.s * a.n_units + cc.unit] =
          a.part_tiles > 0 ? make_int2(cc.p0, wk.parts_of(cc.nt)) : make_int2(w, wk.wave_of_last(cc));
    // Wait for the q rows here, once per piece.  Left to the compiler, the wait lands at
    // the first use of q on every tile (it cannot tell whether this branch ran) and would
    // drain the K/V loads in flight each time.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  // Scores, softmax update and P.V for one tile with cn valid tokens.  Scores stay in
  // raw dot-product units; the probability of score x is exp2(x * scale_log2 - m), with
  // m the piece's reference (log2 units).  The reference is raised only when a score
  // would exceed it by more than kRebase: the probabilities then stay below 2^kRebase,
  // far from overflow, and the costly rescale of the accumulators is rare.  Any
  // reference gives the same result, because every merge rescales by the stored one.
  auto consume = [&](int cn, const u32x4 (&kb)[RK][NL], u32x4 (&vb)[RK][NL]) {
    constexpr float kRebase = 8.0f;
    bool valid[RK];
    const bool full = cn >= TK;  // wave-uniform
#pragma unroll
    for (int r = 0; r < RK; ++r) valid[r] = full || (r * GR + grp < cn);
    if (!full) {  // rows past the context: their V (poison or block 0) must not reach acc
#pragma unroll
      for (int r = 0; r < RK; ++r)
#pragma unroll
        for (int j = 0; j < NL; ++j)
          if (!valid[r]) vb[r][j] = u32x4{0u, 0u, 0u, 0u};
    }
    float sc[GT][RK];
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int r = 0; r < RK; ++r) {
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < NL; ++j) d = dot16<T>(qv[g][j], kb[r][j], d);
        sc[g][r] = group_sum<C>(d);
      }
    float mt[GT];
    bool need = false;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      mt[g] = -INFINITY;
#pragma unroll
      for (int r = 0; r < RK; ++r) mt[g] = fmaxf(mt[g], valid[r] ? sc[g][r] : -INFINITY);
      mt[g] *= a.scale_log2;  // scale > 0: the largest raw score gives the largest scaled one
      need |= mt[g] > m[g] + kRebase;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float m_new = fmaxf(m[g], mt[g]);
        const float corr = rescale(m[g], m_new);
        l[g] *= corr;
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[g][e] *= corr;
        m[g] = m_new;
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int r = 0; r < RK; ++r) {
        const float p = valid[r] ? __builtin_amdgcn_exp2f(fmaf(sc[g][r], a.scale_log2, -m[g])) : 0.0f;
        l[g] += p;
        PV<T>::template run<NL>(acc[g], p, vb[r]);
      }
  };

  // fold another token group's running state (max mo, sum lo, output acco) into row g
  auto merge_state = [&](int g, float mo, float lo, const float* acco) {
    const float mm = fmaxf(m[g], mo);
    const float ca = rescale(m[g], mm);
    const float cb = rescale(mo, mm);
    l[g] = l[g] * ca + lo * cb;
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[g][e] = acc[g][e] * ca + acco[e] * cb;
    m[g] = mm;
  };
  // the same across a row-swap permute, which hands every lane both halves' values
  auto merge_swapped = [&](int g, bool use32) {
    float lo_acc[DL], hi_acc[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      const auto ax = use32 ? __builtin_amdgcn_permlane32_swap(as_u(acc[g][e]), as_u(acc[g][e]), false, false)
                            : __builtin_amdgcn_permlane16_swap(as_u(acc[g][e]), as_u(acc[g][e]), false, false);
      lo_acc[e] = as_f(ax[0]);
      hi_acc[e] = as_f(ax[1]);
    }
    const auto mx = use32 ? __builtin_amdgcn_permlane32_swap(as_u(m[g]), as_u(m[g]), false, false)
                          : __builtin_amdgcn_permlane16_swap(as_u(m[g]), as_u(m[g]), false, false);
    const auto lx = use32 ? __builtin_amdgcn_permlane32_swap(as_u(l[g]), as_u(l[g]), false, false)
                          : __builtin_amdgcn_permlane16_swap(as_u(l[g]), as_u(l[g]), false, false);
    m[g] = as_f(mx[0]);
    l[g] = as_f(lx[0]);
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[g][e] = lo_acc[e];
    merge_state(g, as_f(mx[1]), as_f(lx[1]), hi_acc);
  };

  // finish the piece that ends with the current tile: merge the token groups, then write
  // the rows (a segment this wave holds whole, or of one partition) or a piece record
  auto piece_end = [&]() {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      if constexpr (C == 8) {  // the two token groups of each 16-lane row
        float other[DL];
#pragma unroll
        for (int e = 0; e < DL; ++e) other[e] = dpp_f<0x128>(acc[g][e]);  // row_ror:8
        merge_state(g, dpp_f<0x128>(m[g]), dpp_f<0x128>(l[g]), other);
      }
      merge_swapped(g, true);   // lanes i and i^32
      merge_swapped(g, false);  // lanes i and i^16
    }
    // lanes 0..C-1 now hold the piece's state for their chunks of the row
    if (grp != 0) return;
    // with partitions, a record per partition; rows only for a context of one partition
    const bool part = a.part_tiles > 0;
    const bool whole = part ? wk.parts_of(cc.nt) == 1 : cc.gstart >= A && cc.gstart + cc.nt <= A_end;
    const bool head = cc.gstart < A;  // the segment began in an earlier wave
    const float qnan = __builtin_nanf("");
    const int64_t row0 = static_cast<int64_t>(cc.s) * a.num_q_heads + h0;
    const int rec = part ? wk.part_record(cc) : w * 2 + (head ? 0 : 1);
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      if (g >= ng) break;
      const float inv = piece_bad ? qnan : 1.0f / l[g];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = acc[g][j * E + e] * inv;
        const int col = (j * C + sub) * E;
        if (whole) {
          *reinterpret_cast<u32x4*>(static_cast<T*>(a.out) + (row0 + g) * D + col) = pack16<T>(o);
        } else {
          float* dst = a.rec_o + (static_cast<int64_t>(rec) * a.rec_rows + g) * D + col;
#pragma unroll
          for (int e = 0; e < E; e += 4)
            *reinterpret_cast<u32x4*>(dst + e) = pack16<float>(&o[e]);
        }
      }
      if (!whole && sub == 0) {
        a.rec_m[rec * a.rec_rows + g] = piece_bad ? qnan : m[g];
        a.rec_l[rec * a.rec_rows + g] = piece_bad ? qnan : l[g];
      }
    }
  };

  auto process = [&](int i, const u32x4 (&kb)[RK][NL], u32x4 (&vb)[RK][NL], bool stage_bad) {
    if (i == 0 || wk.piece_starts(cc)) piece_start();
    piece_bad |= stage_bad;
    consume(min(TK, cc.ctx - cc.t * TK), kb, vb);
    if (i == n_my - 1 || wk.piece_ends(cc)) piece_end();
    advance(cc);
  };

  // ---- main loop: the fetch cursor runs two tiles ahead of the compute cursor; every
  // round issues the same loads (phantom tiles past the share read block 0)
  Cursor cf = cc;
  u32x4 k0[RK][NL], v0[RK][NL], k1[RK][NL], v1[RK][NL];
  bool fb0 = fetch(cf, 0 < n_my, 0);
  advance(cf);
  bool fb1 = fetch(cf, 1 < n_my, 1);
  advance(cf);
  unstage(0, k0, v0);
  bool pb0 = fb0;
  fb0 = fetch(cf, 2 < n_my, 0);
  advance(cf);
  for (int i = 0; i < n_my; i += 2) {
    process(i, k0, v0, pb0);
    unstage(1, k1, v1);
    const bool pb1 = fb1;
    fb1 = fetch(cf, i + 3 < n_my, 1);
    advance(cf);
    if (i + 1 < n_my) process(i + 1, k1, v1, pb1);
    unstage(0, k0, v0);
    pb0 = fb0;
    fb0 = fetch(cf, i + 4 < n_my, 0);
    advance(cf);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load still writes LDS at exit
}

// ---------------------------------------------------------------------------
// fp16 decode, pass 1, on the matrix cores
//
// Per tile of 16 tokens, with K and V staged in LDS:
//   S^T = K Q^T       D/32 v_mfma_f32_16x16x32_f16: A = K (token x dims), B = Q^T
//   O^T += V^T P^T    D/16 v_mfma_f32_16x16x16_f16: A = V^T (dims x token), B = P^T
// The 16 columns of B are the query heads that share the kv head (a group of up to 16;
// unused columns are zero).  Lane (g, j) = (lane % 16, lane / 16) gets scores of row g
// for tokens 4j..4j+3, which is exactly the P^T operand layout of the second product,
// and accumulates O[g][16 nb + 4j + i]: the softmax state of row g stays in the lanes
// of row g.  V^T comes out of LDS through the transposing ds_read_b64_tr_b16.
// ---------------------------------------------------------------------------

typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfRows = 16;  // query rows per wave: the N extent of both products

template <int D, bool F8>
struct MCfg {
  static constexpr int kRowQ = D * 2;          // bytes per fp16 q row
  static constexpr int kNCQ = kRowQ / 16;      // 16-byte chunks per q row
  static constexpr int kRow = F8 ? D : D * 2;  // bytes per K or V token row (E4M3 or fp16)
  static constexpr int kNC = kRow / 16;        // 16-byte chunks per K/V row: 4, 8 or 16
  static constexpr int kTK = 16;               // tokens per tile
  static constexpr int kHalf = kTK * kRow;     // bytes of K (or V) per tile
  static constexpr int kLoads = kHalf / 1024;  // 1 KB direct-to-LDS loads for each of K and V
  static constexpr int kKB = D / 32;           // products for the scores
  static constexpr int kNB = D / 16;           // products for P.V
  static constexpr int kQ = kMfRows * kRowQ;     // q rows of a piece (at most 16)
  static constexpr int kStage = 2 * kHalf + kQ;  // one ring stage: K tile, V tile, q rows
  static constexpr int kRowsPerLoad = 64 / kNC;
  static_assert(kLoads * kRowsPerLoad == kTK, "a load covers whole rows");
};

// Chunk c of token row r is stored at chunk position c ^ swz(r) of that row.  Over any 8
// consecutive rows swz takes 8 distinct values, so the 8 lanes of one ds_read_b128 cycle
// (rows 0-7 or 8-15, one chunk) hit distinct banks; over each aligned group of 4 rows
// swz / 2 takes 4 distinct values, so the 16 lanes of one transposing read cycle (4 rows
// x 2 chunks) do too.
__device__ __forceinline__ int swz(int r) { return (2 * r + (r >> 2)) & 7; }

// Chunk position of chunk 0 of key row r (mod 16) in a ring of 256-byte rows: chunk c is stored
// at c ^ swz16(r).  D = 128 rows are 256 bytes, a full sweep of the LDS banks.  swz16 is a
// permutation of 0..15, so the 16 rows a 16-lane quarter of a ds_read_b128 reads (one chunk
// each) land on 16 distinct positions; and the transposing V reads, 2 adjacent chunks of 4
// rows per 16 lanes, cover 8 distinct positions per 4-row group and all 16 over rows 0-7
// (and 8-15), conflict-free whether the LDS serves 16 or 32 lanes of them per cycle.
// D = 64 rows are 128 bytes: swz already keeps even rows, and odd rows, apart.
template <int D>
__device__ __forceinline__ int swz16(int r) {
  if constexpr (D == 128) return 2 * (r & 3) + 8 * ((r >> 2) & 1) + ((r >> 3) & 1);
  return swz(r);
}

// A wave-uniform pointer, forced into SGPRs (an asm "s" operand needs it there).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Read one ring stage's operands, and load the two block-table entries the next fetch
// needs.  In order: issue the two scalar loads of the entries; wait until at most VM
// vector-memory operations are outstanding (the stage's own loads are older); read the K
// operands (ds_read_b128) and the V^T operands (ds_read_b64_tr_b16) at the lane's
// addresses + OFF; wait for the reads and the entries (lgkmcnt counts both).  The entry
// loads thus overlap the wait for the stage instead of stalling the fetch.  One asm block,
// so the compiler's conservative tracking of direct-to-LDS loads cannot put a full drain
// in front of the reads.  Outputs are early-clobber: the reads complete asynchronously,
// so no output may share a register with an address still to be read.
template <int VM, int OFF>
__device__ __forceinline__ void read_stage_d128(const uint32_t (&ka)[4], const uint32_t (&va)[8],
                                                f16x8 (&k)[4], f16x4 (&v)[8], const int32_t* e0,
                                                const int32_t* e1, int32_t& p0, int32_t& p1) {
  asm volatile(
      "s_load_dword %[p0], %[e0], 0x0\n\t"
      "s_load_dword %[p1], %[e1], 0x0\n\t"
      "s_waitcnt vmcnt(%[vm])\n\t"
      "ds_read_b128 %[k0], %[ka0] offset:%[off]\n\t"
      "ds_read_b128 %[k1], %[ka1] offset:%[off]\n\t"
      "ds_read_b128 %[k2], %[ka2] offset:%[off]\n\t"
      "ds_read_b128 %[k3], %[ka3] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v0], %[va0] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v1], %[va1] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v2], %[va2] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v3], %[va3] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v4], %[va4] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v5], %[va5] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v6], %[va6] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v7], %[va7] offset:%[off]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [k2] "=&v"(k[2]), [k3] "=&v"(k[3]), [v0] "=&v"(v[0]),
        [v1] "=&v"(v[1]), [v2] "=&v"(v[2]), [v3] "=&v"(v[3]), [v4] "=&v"(v[4]), [v5] "=&v"(v[5]),
        [v6] "=&v"(v[6]), [v7] "=&v"(v[7]), [p0] "=&s"(p0), [p1] "=&s"(p1)
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [ka2] "v"(ka[2]), [ka3] "v"(ka[3]), [va0] "v"(va[0]),
        [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]), [va4] "v"(va[4]), [va5] "v"(va[5]),
        [va6] "v"(va[6]), [va7] "v"(va[7]), [e0] "s"(e0), [e1] "s"(e1), [vm] "n"(VM), [off] "n"(OFF)
      : "memory");
}

template <int VM, int OFF>
__device__ __forceinline__ void read_stage_d64(const uint32_t (&ka)[2], const uint32_t (&va)[4],
                                               f16x8 (&k)[2], f16x4 (&v)[4], const int32_t* e0,
                                               const int32_t* e1, int32_t& p0, int32_t& p1) {
  asm volatile(
      "s_load_dword %[p0], %[e0], 0x0\n\t"
      "s_load_dword %[p1], %[e1], 0x0\n\t"
      "s_waitcnt vmcnt(%[vm])\n\t"
      "ds_read_b128 %[k0], %[ka0] offset:%[off]\n\t"
      "ds_read_b128 %[k1], %[ka1] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v0], %[va0] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v1], %[va1] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v2], %[va2] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v3], %[va3] offset:%[off]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [v0] "=&v"(v[0]), [v1] "=&v"(v[1]), [v2] "=&v"(v[2]),
        [v3] "=&v"(v[3]), [p0] "=&s"(p0), [p1] "=&s"(p1)
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]),
        [va3] "v"(va[3]), [e0] "s"(e0), [e1] "s"(e1), [vm] "n"(VM), [off] "n"(OFF)
      : "memory");
}

// The same reads for the virtually contiguous cache, which has no table entries to load.
template <int VM, int OFF>
__device__ __forceinline__ void read_stage_d128_dense(const uint32_t (&ka)[4], const uint32_t (&va)[8],
                                                      f16x8 (&k)[4], f16x4 (&v)[8]) {
  asm volatile(
      "s_waitcnt vmcnt(%[vm])\n\t"
      "ds_read_b128 %[k0], %[ka0] offset:%[off]\n\t"
      "ds_read_b128 %[k1], %[ka1] offset:%[off]\n\t"
      "ds_read_b128 %[k2], %[ka2] offset:%[off]\n\t"
      "ds_read_b128 %[k3], %[ka3] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v0], %[va0] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v1], %[va1] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v2], %[va2] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v3], %[va3] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v4], %[va4] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v5], %[va5] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v6], %[va6] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v7], %[va7] offset:%[off]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [k2] "=&v"(k[2]), [k3] "=&v"(k[3]), [v0] "=&v"(v[0]),
        [v1] "=&v"(v[1]), [v2] "=&v"(v[2]), [v3] "=&v"(v[3]), [v4] "=&v"(v[4]), [v5] "=&v"(v[5]),
        [v6] "=&v"(v[6]), [v7] "=&v"(v[7])
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [ka2] "v"(ka[2]), [ka3] "v"(ka[3]), [va0] "v"(va[0]),
        [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]), [va4] "v"(va[4]), [va5] "v"(va[5]),
        [va6] "v"(va[6]), [va7] "v"(va[7]), [vm] "n"(VM), [off] "n"(OFF)
      : "memory");
}

template <int VM, int OFF>
__device__ __forceinline__ void read_stage_d64_dense(const uint32_t (&ka)[2], const uint32_t (&va)[4],
                                                     f16x8 (&k)[2], f16x4 (&v)[4]) {
  asm volatile(
      "s_waitcnt vmcnt(%[vm])\n\t"
      "ds_read_b128 %[k0], %[ka0] offset:%[off]\n\t"
      "ds_read_b128 %[k1], %[ka1] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v0], %[va0] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v1], %[va1] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v2], %[va2] offset:%[off]\n\t"
      "ds_read_b64_tr_b16 %[v3], %[va3] offset:%[off]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [v0] "=&v"(v[0]), [v1] "=&v"(v[1]), [v2] "=&v"(v[2]),
        [v3] "=&v"(v[3])
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]),
        [va3] "v"(va[3]), [vm] "n"(VM), [off] "n"(OFF)
      : "memory");
}

template <int D, int VM, int OFF>
__device__ __forceinline__ void read_stage_mf(const uint32_t (&ka)[D / 32], const uint32_t (&va)[D / 16],
                                              f16x8 (&k)[D / 32], f16x4 (&v)[D / 16], const int32_t* e0,
                                              const int32_t* e1, int32_t& p0, int32_t& p1) {
  if constexpr (D == 128) read_stage_d128<VM, OFF>(ka, va, k, v, e0, e1, p0, p1);
  else read_stage_d64<VM, OFF>(ka, va, k, v, e0, e1, p0, p1);
}

// ---- E4M3 pools ([CON] section 6: blocks hold compressed K/V that the kernel expands)
//
// A row of D codes is D bytes.  The products still run in fp16: every E4M3 value is an
// fp16 value, so the conversion is exact, and the K and V scales are applied in fp32
// (K's folded into the score scale, V's into the final normalisation).  Token order
// within a tile differs from the fp16 kernel: lane quarter jq holds tokens jq, jq + 4,
// jq + 8, jq + 12 (tau below), so that the V rows one 16-lane phase reads are adjacent.
// V^T is built in registers: a lane reads, for each of its four tokens, the NB codes of
// dims NB g .. NB g + NB - 1 (one 8- or 4-byte read), and a byte transpose turns them
// into the NB operands {token 0..3} of one dim each.

// Token of a tile held in score row i (the K row lane g reads is tau(g)).
__device__ __forceinline__ int tau(int i) { return (i >> 2) + 4 * (i & 3); }

// Chunk c of E4M3 row r is stored at chunk position c ^ swz8<D>(r).  A 16-lane quarter of
// a ds_read_b128 reads one chunk of all 16 rows of a tile.  D = 128 rows are 128 bytes, so
// even rows fall on one half of the 64 banks and odd rows on the other: swz8 takes 8
// distinct values over the even rows and over the odd rows (and over rows tau(0..7) and
// tau(8..15), the rows 8 lanes read together).  D = 64 rows are 64 bytes, a quarter of the
// banks each: swz8 takes 4 distinct values over the rows of each quarter.
template <int D>
__device__ __forceinline__ int swz8(int r) {
  return D == 128 ? (((r >> 1) & 7) ^ (r & 1)) : ((r >> 2) & 3);
}

// Four E4M3 codes (byte i = element i) as fp16, exactly.
__device__ __forceinline__ f16x4 e4m3x4_to_f16(uint32_t x) {
  const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  return f16x4{lo[0], lo[1], hi[0], hi[1]};
}

// 4 x 4 byte transpose: byte j of w[i] = byte i of x[j].  v_perm_b32 picks bytes 0-3
// from its second source and 4-7 from its first.
__device__ __forceinline__ void byte_transpose4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                                uint32_t (&w)[4]) {
  const uint32_t a_lo = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0.0 x1.0 x0.1 x1.1
  const uint32_t a_hi = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0.2 x1.2 x0.3 x1.3
  const uint32_t b_lo = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
  const uint32_t b_hi = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
  w[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
  w[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
  w[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
  w[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

// The E4M3 stage read: like read_stage_d128, with the K codes in two ds_read_b128 and
// the V codes of the lane's four tokens in four ds_read_b64 (D = 128), or one
// ds_read_b128 and four ds_read_b32 (D = 64).
template <int VM, int OFF>
__device__ __forceinline__ void read_stage_f8_d128(const uint32_t (&ka)[2], const uint32_t (&va)[4],
                                                   u32x4 (&k)[2], u32x2 (&v)[4], const int32_t* e0,
                                                   const int32_t* e1, int32_t& p0, int32_t& p1) {
  asm volatile(
      "s_load_dword %[p0], %[e0], 0x0\n\t"
      "s_load_dword %[p1], %[e1], 0x0\n\t"
      "s_waitcnt vmcnt(%[vm])\n\t"
      "ds_read_b128 %[k0], %[ka0] offset:%[off]\n\t"
      "ds_read_b128 %[k1], %[ka1] offset:%[off]\n\t"
      "ds_read_b64 %[v0], %[va0] offset:%[off]\n\t"
      "ds_read_b64 %[v1], %[va1] offset:%[off]\n\t"
      "ds_read_b64 %[v2], %[va2] offset:%[off]\n\t"
      "ds_read_b64 %[v3], %[va3] offset:%[off]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [v0] "=&v"(v[0]), [v1] "=&v"(v[1]), [v2] "=&v"(v[2]),
        [v3] "=&v"(v[3]), [p0] "=&s"(p0), [p1] "=&s"(p1)
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]),
        [va3] "v"(va[3]), [e0] "s"(e0), [e1] "s"(e1), [vm] "n"(VM), [off] "n"(OFF)
      : "memory");
}

template <int VM, int OFF>
__device__ __forceinline__ void read_stage_f8_d64(const uint32_t (&ka)[1], const uint32_t (&va)[4],
                                                  u32x4 (&k)[1], uint32_t (&v)[4], const int32_t* e0,
                                                  const int32_t* e1, int32_t& p0, int32_t& p1) {
  asm volatile(
      "s_load_dword %[p0], %[e0], 0x0\n\t"
      "s_load_dword %[p1], %[e1], 0x0\n\t"
      "s_waitcnt vmcnt(%[vm])\n\t"
      "ds_read_b128 %[k0], %[ka0] offset:%[off]\n\t"
      "ds_read_b32 %[v0], %[va0] offset:%[off]\n\t"
      "ds_read_b32 %[v1], %[va1] offset:%[off]\n\t"
      "ds_read_b32 %[v2], %[va2] offset:%[off]\n\t"
      "ds_read_b32 %[v3], %[va3] offset:%[off]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k0] "=&v"(k[0]), [v0] "=&v"(v[0]), [v1] "=&v"(v[1]), [v2] "=&v"(v[2]), [v3] "=&v"(v[3]),
        [p0] "=&s"(p0), [p1] "=&s"(p1)
      : [ka0] "v"(ka[0]), [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]),
        [e0] "s"(e0), [e1] "s"(e1), [vm] "n"(VM), [off] "n"(OFF)
      : "memory");
}

// Read an E4M3 stage and expand it into the fp16 operands of the fp16 kernel: kop[kb]
// holds the codes of dims 8 (jq KB + kb) .. + 7 of K row tau(g); vop[nb] holds dim
// NB g + nb of V rows tau(4 jq + t), t = 0..3.
template <int D, int VM, int OFF>
__device__ __forceinline__ void read_stage_f8(const uint32_t (&ka)[D / 64], const uint32_t (&va)[4],
                                              f16x8 (&kop)[D / 32], f16x4 (&vop)[D / 16],
                                              const int32_t* e0, const int32_t* e1, int32_t& p0,
                                              int32_t& p1) {
  u32x4 kr[D / 64];
  uint32_t x[4], y[4];
  if constexpr (D == 128) {
    u32x2 vr[4];
    read_stage_f8_d128<VM, OFF>(ka, va, kr, vr, e0, e1, p0, p1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      x[t] = vr[t][0];
      y[t] = vr[t][1];
    }
  } else {
    read_stage_f8_d64<VM, OFF>(ka, va, kr, x, e0, e1, p0, p1);
  }
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) {
    const f16x4 a = e4m3x4_to_f16(kr[kb / 2][2 * (kb % 2)]);
    const f16x4 b = e4m3x4_to_f16(kr[kb / 2][2 * (kb % 2) + 1]);
    kop[kb] = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  uint32_t w[4];
  byte_transpose4(x[0], x[1], x[2], x[3], w);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) vop[nb] = e4m3x4_to_f16(w[nb]);
  if constexpr (D == 128) {
    byte_transpose4(y[0], y[1], y[2], y[3], w);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) vop[4 + nb] = e4m3x4_to_f16(w[nb]);
  }
}

// Six wave-uniform 32-bit loads through the scalar unit with a single wait.
__device__ __forceinline__ void load_entries6(const int32_t* a0, const int32_t* a1, const int32_t* a2,
                                              const int32_t* a3, const int32_t* a4, const int32_t* a5,
                                              int32_t (&p)[6]) {
  asm volatile(
      "s_load_dword %[p0], %[a0], 0x0\n\t"
      "s_load_dword %[p1], %[a1], 0x0\n\t"
      "s_load_dword %[p2], %[a2], 0x0\n\t"
      "s_load_dword %[p3], %[a3], 0x0\n\t"
      "s_load_dword %[p4], %[a4], 0x0\n\t"
      "s_load_dword %[p5], %[a5], 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [p0] "=&s"(p[0]), [p1] "=&s"(p[1]), [p2] "=&s"(p[2]), [p3] "=&s"(p[3]), [p4] "=&s"(p[4]),
        [p5] "=&s"(p[5])
      : [a0] "s"(a0), [a1] "s"(a1), [a2] "s"(a2), [a3] "s"(a3), [a4] "s"(a4), [a5] "s"(a5)
      : "memory");
}

// Two wave-uniform 32-bit loads through the scalar unit with a single wait.
__device__ __forceinline__ void load_entries2(const int32_t* a0, const int32_t* a1, int32_t (&p)[2]) {
  asm volatile(
      "s_load_dword %[p0], %[a0], 0x0\n\t"
      "s_load_dword %[p1], %[a1], 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [p0] "=&s"(p[0]), [p1] "=&s"(p[1])
      : [a0] "s"(a0), [a1] "s"(a1)
      : "memory");
}

// Four wave-uniform 32-bit loads through the scalar unit with a single wait.
__device__ __forceinline__ void load_entries4(const int32_t* a0, const int32_t* a1, const int32_t* a2,
                                              const int32_t* a3, int32_t (&p)[4]) {
  asm volatile(
      "s_load_dword %[p0], %[a0], 0x0\n\t"
      "s_load_dword %[p1], %[a1], 0x0\n\t"
      "s_load_dword %[p2], %[a2], 0x0\n\t"
      "s_load_dword %[p3], %[a3], 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [p0] "=&s"(p[0]), [p1] "=&s"(p[1]), [p2] "=&s"(p[2]), [p3] "=&s"(p[3])
      : [a0] "s"(a0), [a1] "s"(a1), [a2] "s"(a2), [a3] "s"(a3)
      : "memory");
}

// Eight fp16 values, each replaced by the fp16 value of the E4M3 code the store gives it
// with scale sc.
__device__ __forceinline__ f16x8 e4m3_values8(const u32x4& x, F8Scale sc) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f16x2 h = word_as<f16x2>(x, i / 2);
    float val;
    (void)e4m3_code_exact(static_cast<float>(h[i % 2]), sc, val);
    r[i] = static_cast<f16>(val);
  }
  return r;
}

// E4M3 append mode: read the new token's fp16 rows from a stage's new-row area (K row at
// OFF, V row at OFF + 2 D): k[kb] = the 8 K values of dims 8 (jq KB + kb) .. + 7 (at the
// lane's address nk + 16 kb), v = the NB V values of dims NB g .. NB g + NB - 1 (at nv;
// D = 64 fills the low half).  asm for the same reason as the stage reads.
template <int D, int OFF>
__device__ __forceinline__ void read_new_rows_f8(uint32_t nk, uint32_t nv, u32x4 (&k)[D / 32], u32x4& v) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %[k0], %[a] offset:%[o0]\n\t"
        "ds_read_b128 %[k1], %[a] offset:%[o1]\n\t"
        "ds_read_b128 %[k2], %[a] offset:%[o2]\n\t"
        "ds_read_b128 %[k3], %[a] offset:%[o3]\n\t"
        "ds_read_b128 %[v0], %[b] offset:%[ov]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [k2] "=&v"(k[2]), [k3] "=&v"(k[3]), [v0] "=&v"(v)
        : [a] "v"(nk), [b] "v"(nv), [o0] "n"(OFF), [o1] "n"(OFF + 16), [o2] "n"(OFF + 32),
          [o3] "n"(OFF + 48), [ov] "n"(OFF + 2 * D)
        : "memory");
  } else {
    static_assert(D == 64, "head_dim");
    u32x2 h;
    asm volatile(
        "ds_read_b128 %[k0], %[a] offset:%[o0]\n\t"
        "ds_read_b128 %[k1], %[a] offset:%[o1]\n\t"
        "ds_read_b64 %[v0], %[b] offset:%[ov]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [v0] "=&v"(h)
        : [a] "v"(nk), [b] "v"(nv), [o0] "n"(OFF), [o1] "n"(OFF + 16), [ov] "n"(OFF + 2 * D)
        : "memory");
    v = u32x4{h[0], h[1], 0u, 0u};
  }
}

// Read a piece's q operand from LDS: chunks kb = 0 .. KB-1 at the lane's address + OFF +
// 16 kb.  Called after the stage wait that covers the q loads; asm for the same reason
// as the stage reads.
template <int KB, int OFF>
__device__ __forceinline__ void read_q_mf(uint32_t addr, f16x8 (&q)[KB]) {
  if constexpr (KB == 4) {
    asm volatile(
        "ds_read_b128 %[q0], %[a] offset:%[o0]\n\t"
        "ds_read_b128 %[q1], %[a] offset:%[o1]\n\t"
        "ds_read_b128 %[q2], %[a] offset:%[o2]\n\t"
        "ds_read_b128 %[q3], %[a] offset:%[o3]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [q0] "=&v"(q[0]), [q1] "=&v"(q[1]), [q2] "=&v"(q[2]), [q3] "=&v"(q[3])
        : [a] "v"(addr), [o0] "n"(OFF), [o1] "n"(OFF + 16), [o2] "n"(OFF + 32), [o3] "n"(OFF + 48)
        : "memory");
  } else {
    static_assert(KB == 2, "q chunks per lane");
    asm volatile(
        "ds_read_b128 %[q0], %[a] offset:%[o0]\n\t"
        "ds_read_b128 %[q1], %[a] offset:%[o1]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [q0] "=&v"(q[0]), [q1] "=&v"(q[1])
        : [a] "v"(addr), [o0] "n"(OFF), [o1] "n"(OFF + 16)
        : "memory");
  }
}

// Call f(std::integral_constant<int, i>{}) for i = 0 .. N-1: a loop whose index is a
// compile-time constant in the body (stage offsets become instruction immediates).
template <typename F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// F8: E4M3 pools.  DENSE: the virtually contiguous cache of pa_decode_dense (fp16, no table).
// APPEND: each sequence's newest token (position ctx - 1) comes from a.k_new / a.v_new (fp16
// rows), not from the pools, which the same call writes only after this kernel
// (pa_decode_append, pa_decode_fp8_append).  fp16 pools load that row in place of the
// pool's; E4M3 pools stage the fp16 rows beside the tile and replace the token's operands
// with the values of their codes.
template <int D, int NST, bool F8, bool DENSE = false, bool APPEND = false>
__global__ __launch_bounds__(kWave) void pa_stream_mfma_kernel(const StreamArgs a) {
  static_assert(!(F8 && DENSE), "the contiguous cache is fp16");
  static_assert(!(APPEND && DENSE), "append mode reads the pools");
  using K = MCfg<D, F8>;
  constexpr int TK = K::kTK, KB = K::kKB, NB = K::kNB, NC = K::kNC, ROW = K::kRow;
  constexpr int ROWQ = K::kRowQ, NCQ = K::kNCQ;
  constexpr int LOADS = K::kLoads, HALF = K::kHalf;
  constexpr bool F8NEW = APPEND && F8;  // E4M3 append: the new fp16 rows get a stage area
  constexpr int NEWOFF = K::kStage;     // K row (2 D bytes), then V row
  constexpr int STAGE = F8NEW ? (K::kStage + 4 * D + 1023) / 1024 * 1024 : K::kStage;
  constexpr int QOFF = 2 * HALF;             // q rows within a stage
  constexpr int QROWS = 1024 / ROWQ;         // q rows per 1 KB load
  constexpr int KR = D / 64;                 // E4M3: 16-byte K reads per lane
  constexpr int VM = (NST - 1) * 2 * LOADS;  // loads younger than a stage when it is read
  static_assert(VM <= 63, "vmcnt range");
  static_assert(NST * STAGE <= 65536, "stage offsets are 16-bit immediates");
  __shared__ __align__(1024) char s_ring[NST * STAGE];

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int g = lane % 16;   // query row (column of the products)
  const int jq = lane / 16;  // token quarter: tokens 4 jq .. 4 jq + 3 of a tile

  Work<TK> wk;
  Cursor cc;
  wk.init(a, w, lane, cc);
  const int n_my = wk.n_my;
  if (n_my == 0) return;
  const int A = wk.A, A_end = A + n_my;

  // ---- per-lane LDS addresses (within a stage) of the operands, and of the loads
  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s_ring));
  constexpr int NKA = F8 ? KR : KB, NVA = F8 ? 4 : NB;
  uint32_t ka[NKA], va[NVA];
  if constexpr (F8) {
    const int rk = tau(g);  // lane (g, jq) takes dims 8 jq KB .. 8 jq KB + 8 KB - 1 of row tau(g)
#pragma unroll
    for (int j = 0; j < KR; ++j)
      ka[j] = ring + static_cast<uint32_t>(rk * ROW + (((jq * KR + j) ^ swz8<D>(rk)) * 16));
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // row tau(4 jq + t) = jq + 4 t, dims NB g .. NB g + NB - 1
      const int r = jq + 4 * t;
      const int byte = NB * g;
      va[t] = ring + static_cast<uint32_t>(HALF + r * ROW + (((byte >> 4) ^ swz8<D>(r)) * 16) + (byte & 15));
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {  // lane (g = token, jq) takes chunk jq * KB + kb of row g
      const int c = jq * KB + kb;
      ka[kb] = ring + static_cast<uint32_t>(g * ROW + ((c ^ swz16<D>(g)) * 16));
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {  // lane 16 jq + 4 i + q: row 4 jq + i, dims 16 nb + 4 q
      const int r = 4 * jq + (g >> 2), q = g & 3;
      const int c = 2 * nb + (q >> 1);
      va[nb] = ring + static_cast<uint32_t>(HALF + r * ROW + ((c ^ swz16<D>(r)) * 16) + (q & 1) * 8);
    }
  }
  // q operand: lane (g, jq) reads chunks jq * KB .. jq * KB + KB - 1 of q row g
  const uint32_t qa = ring + static_cast<uint32_t>(g * ROWQ + jq * KB * 16);
  // load i, lane l fills LDS position 64 i + l of a half: row r, chunk position p, which
  // holds chunk p ^ swz16(r) of the row; lo[i] is its byte offset from the row slot start,
  // hi8[i] whether the row is in the second half of the tile
  const int bsz = a.block_size;
  uint32_t lo[LOADS];
  bool hi8[LOADS];
  int row_of[LOADS];         // append mode: the tile row of load i, and the offset of its
  uint32_t chunk_of[LOADS];  // chunk within a row
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = i * 64 + lane;
    const int r = pos / NC, p = pos % NC;
    const int rr = bsz >= TK ? r : (r & (bsz - 1));  // row within its block
    const int sw = F8 ? swz8<D>(r) : swz16<D>(r);
    row_of[i] = r;
    chunk_of[i] = static_cast<uint32_t>((p ^ sw) * 16);
    // contiguous cache: consecutive tokens of one head are token_bytes apart
    lo[i] = DENSE ? static_cast<uint32_t>(r * a.token_bytes + ((p ^ sw) * 16))
                  : static_cast<uint32_t>(rr * ROW + ((p ^ sw) * 16));
    hi8[i] = r >= 8;
  }

  const char* kcache = static_cast<const char*>(a.k_cache);
  const char* vcache = static_cast<const char*>(a.v_cache);
  const char* qbytes = static_cast<const char*>(a.q);
  const uint64_t head_bytes = static_cast<uint64_t>(bsz) * ROW;
  const uint64_t block_bytes = head_bytes * static_cast<uint64_t>(a.num_kv_heads);

  // Block-table entries of tile f: the first row slot's, and for block size 8 the second
  // half's (the first again when that half lies past the context).  A phantom tile past
  // the share points at entry 0 of row 0, a valid address whose value is not used.
  auto entry_ptrs = [&](const Cursor& f, bool real, const int32_t*& e0, const int32_t*& e1)
      __attribute__((always_inline)) {
    if (!real) {
      e0 = e1 = uniform_ptr(a.block_tables);
      return;
    }
    const int tok0 = f.t * TK;
    const int32_t* p = a.block_tables + static_cast<int64_t>(f.s) * a.max_blocks_per_seq +
                       (tok0 >> a.log2_block);
    e0 = uniform_ptr(p);
    e1 = (bsz < TK && tok0 + bsz < f.ctx) ? uniform_ptr(p + 1) : e0;
  };

  // Issue the loads of tile f into stage st, given its table entries p0, p1: first the q
  // rows of the piece when the tile starts one (qload), then K and V.  A tile spans one
  // block for block sizes 16 and 32 and two for block size 8 (rows 0-7 and 8-15).  Phantom
  // tiles past the share read block 0, and so do row slots past the context: valid
  // addresses, data unused.  Returns whether an entry lies outside the pool.
  auto fetch = [&](const Cursor& f, bool real, bool qload, int st, int p0, int p1)
      __attribute__((always_inline)) -> bool {
    bool bad = false;
    const int kvh = real ? f.unit / a.n_gtiles : 0;
    const int tok0 = f.t * TK;
    if (DENSE) {
    } else if (real) {
      if (p0 < 0 || p0 >= a.num_blocks) {
        bad = true;
        p0 = 0;
      }
      if (bsz < TK && tok0 + bsz < f.ctx) {
        if (p1 < 0 || p1 >= a.num_blocks) {
          bad = true;
          p1 = 0;
        }
      } else {
        p1 = 0;
      }
    } else {
      p0 = 0;
      p1 = 0;
    }
    char* stage = s_ring + st * STAGE;
    if (qload) {  // wave-uniform: rows h0 .. h0 + ng - 1 of the piece's sequence
      const int gtile = f.unit - kvh * a.n_gtiles;
      const int h0 = kvh * a.group + gtile * kMfRows;
      const int ng = min(kMfRows, a.group - gtile * kMfRows);
      const char* qrow0 = qbytes + (static_cast<int64_t>(f.s) * a.num_q_heads + h0) * ROWQ;
#pragma unroll
      for (int i = 0; i < kMfRows / QROWS; ++i) {
        if (i * QROWS < ng) {
          const int r = min(i * QROWS + lane / NCQ, ng - 1);
          __builtin_amdgcn_global_load_lds(qrow0 + r * ROWQ + (lane % NCQ) * 16, stage + QOFF + i * 1024,
                                           16, 0, 0);
        }
      }
    }
    if constexpr (DENSE) {  // a tile never leaves the page that holds its first token
      const int64_t off = static_cast<int64_t>(f.s) * a.seq_bytes + static_cast<int64_t>(tok0) * a.token_bytes +
                          static_cast<int64_t>(kvh) * ROW;
      const char* kt = real ? a.dense_k + off : a.guard_k;
      const char* vt = real ? a.dense_v + off : a.guard_v;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(kt + lo[i]), static_cast<void*>(stage + i * 1024),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(vt + lo[i]),
                                         static_cast<void*>(stage + HALF + i * 1024), 16, 0, 0);
      }
      return bad;
    }
    const uint64_t head = static_cast<uint64_t>(kvh) * head_bytes;
    const uint64_t b0 = static_cast<uint64_t>(static_cast<uint32_t>(p0)) * block_bytes + head +
                        static_cast<uint64_t>(tok0 & (bsz - 1)) * ROW;
    const uint64_t b1 = static_cast<uint64_t>(static_cast<uint32_t>(p1)) * block_bytes + head;
    if constexpr (F8NEW) {
      // the context's last tile: its new K and V rows (fp16, 16-byte chunks) go to the stage's
      // new-row area, one chunk per lane, ahead of the tile's loads so that the same stage
      // wait covers them
      constexpr int NCN = 2 * D / 16;
      if (real && tok0 + TK >= f.ctx && lane < 2 * NCN) {
        const int64_t nrow = (static_cast<int64_t>(f.s) * a.num_kv_heads + kvh) * (2 * D);
        const char* src = (lane < NCN ? a.k_new : a.v_new) + nrow + (lane % NCN) * 16;
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), static_cast<void*>(stage + NEWOFF), 16, 0,
                                         0);
      }
    }
    if constexpr (APPEND && !F8) {
      if (real && tok0 + TK >= f.ctx) {  // the context's last tile: row ctx - 1 - tok0 is new
        const int rn = f.ctx - 1 - tok0;
        const int64_t nrow = (static_cast<int64_t>(f.s) * a.num_kv_heads + kvh) * ROW;
        const char* kn = a.k_new + nrow;
        const char* vn = a.v_new + nrow;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const bool second = bsz < TK && (K::kRowsPerLoad > 8 ? hi8[i] : i * K::kRowsPerLoad >= 8);
          const uint64_t off = (second ? b1 : b0) + lo[i];
          const bool mine = row_of[i] == rn;
          const char* kp = mine ? kn + chunk_of[i] : kcache + off;
          const char* vp = mine ? vn + chunk_of[i] : vcache + off;
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(kp), static_cast<void*>(stage + i * 1024), 16,
                                           0, 0);
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(vp),
                                           static_cast<void*>(stage + HALF + i * 1024), 16, 0, 0);
        }
        return bad;
      }
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      // wave-uniform unless one load spans both halves (16 rows of 64 codes)
      const bool second = bsz < TK && (K::kRowsPerLoad > 8 ? hi8[i] : i * K::kRowsPerLoad >= 8);
      const uint64_t off = (second ? b1 : b0) + lo[i];
      __builtin_amdgcn_global_load_lds(kcache + off, stage + i * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vcache + off, stage + HALF + i * 1024, 16, 0, 0);
    }
    return bad;
  };

  // ---- per-piece state
  f16x8 qop[KB];   // B operand of the scores: lane (g, jq) holds q[g][8 (jq KB + kb) ..]
  f32x4 o[NB];     // lane (g, jq): O[g][16 nb + 4 jq + i]
  float m = -INFINITY, l = 0.0f;  // row g: reference (log2 units) and this lane's exp-sum
  int h0 = 0, ng = 0;
  bool piece_bad = false;

  // Start a piece at the current tile.  qread: the tile starts the wave's share or its
  // segment, and its stage stc holds the segment's q rows (a later partition of the same
  // segment keeps them).
  auto piece_start = [&](auto stc, bool qread) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    if (qread) {
      const int kvh = cc.unit / a.n_gtiles;
      const int gtile = cc.unit - kvh * a.n_gtiles;
      h0 = kvh * a.group + gtile * kMfRows;
      ng = min(kMfRows, a.group - gtile * kMfRows);
      read_q_mf<KB, st * STAGE + QOFF>(qa, qop);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) qop[kb] = g < ng ? qop[kb] : f16x8{};
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    m = -INFINITY;
    l = 0.0f;
    piece_bad = false;
    if (cc.t == 0 && lane == 0)  // where the segment's pieces are: its waves, or its partitions
      a.seg_desc[cc.s * a.n_units + cc.unit] =
          a.part_tiles > 0 ? make_int2(cc.p0, wk.parts_of(cc.nt)) : make_int2(w, wk.wave_of_last(cc));
  };

  auto consume = [&](int cn, const f16x8 (&kop)[KB], f16x4 (&vop)[NB]) __attribute__((always_inline)) {
    constexpr float kRebase = 8.0f;
    // scores: two accumulation chains halve the dependent-product latency
    f32x4 sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb & 1) sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb], qop[kb], sb, 0, 0, 0);
      else sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb], qop[kb], sa, 0, 0, 0);
    }
    const f32x4 sc = sa + sb;
    const bool full = cn >= TK;  // wave-uniform
    bool ok[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ok[i] = full || ((F8 ? tau(4 * jq + i) : 4 * jq + i) < cn);
      mt = fmaxf(mt, ok[i] ? sc[i] : -INFINITY);
    }
    {  // the row maximum over the tile: lanes g, g+16, g+32, g+48
      const auto x32 = __builtin_amdgcn_permlane32_swap(as_u(mt), as_u(mt), false, false);
      mt = fmaxf(as_f(x32[0]), as_f(x32[1]));
      const auto x16 = __builtin_amdgcn_permlane16_swap(as_u(mt), as_u(mt), false, false);
      mt = fmaxf(as_f(x16[0]), as_f(x16[1]));
    }
    mt *= a.scale_log2;  // scale > 0
    if (__builtin_amdgcn_ballot_w64(mt > m + kRebase) != 0) {
      const float m_new = fmaxf(m, mt);
      const float corr = rescale(m, m_new);
      l *= corr;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] *= corr;
      m = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = ok[i] ? __builtin_amdgcn_exp2f(fmaf(sc[i], a.scale_log2, -m)) : 0.0f;
      l += p[i];
    }
    const f16x4 pb = {static_cast<f16>(p[0]), static_cast<f16>(p[1]), static_cast<f16>(p[2]),
                      static_cast<f16>(p[3])};
    if (!full) {  // V rows past the context (poison or block 0) must not reach O
      const uint32_t mlo = (ok[0] ? 0x0000FFFFu : 0u) | (ok[1] ? 0xFFFF0000u : 0u);
      const uint32_t mhi = (ok[2] ? 0x0000FFFFu : 0u) | (ok[3] ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint64_t x = __builtin_bit_cast(uint64_t, vop[nb]);
        x &= (static_cast<uint64_t>(mhi) << 32) | mlo;
        vop[nb] = __builtin_bit_cast(f16x4, x);
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop[nb], pb, o[nb], 0, 0, 0);
  };

  // finish the piece that ends with the current tile: the row's exp-sum over its four
  // lanes, then the rows (a segment this wave holds whole, or of one partition) or a piece
  // record
  auto piece_end = [&]() __attribute__((always_inline)) {
    float lt = l;
    {
      const auto x32 = __builtin_amdgcn_permlane32_swap(as_u(lt), as_u(lt), false, false);
      lt = as_f(x32[0]) + as_f(x32[1]);
      const auto x16 = __builtin_amdgcn_permlane16_swap(as_u(lt), as_u(lt), false, false);
      lt = as_f(x16[0]) + as_f(x16[1]);
    }
    if (g >= ng) return;
    // with partitions, a record per partition; rows only for a context of one partition
    const bool part = a.part_tiles > 0;
    const bool whole = part ? wk.parts_of(cc.nt) == 1 : cc.gstart >= A && cc.gstart + cc.nt <= A_end;
    const bool head = cc.gstart < A;
    const float qnan = __builtin_nanf("");
    const float inv = piece_bad ? qnan : (F8 ? a.out_scale / lt : 1.0f / lt);
    const int64_t row = static_cast<int64_t>(cc.s) * a.num_q_heads + h0 + g;
    const int rec = part ? wk.part_record(cc) : w * 2 + (head ? 0 : 1);
    if constexpr (F8) {
      // o[nb][r] is dim NB (4 jq + r) + nb: the lane holds dims 4 NB jq .. 4 NB jq + 4 NB - 1
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = NB * (4 * jq + r);
        float y[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) y[nb] = o[nb][r] * inv;
        if (whole) {
          f16* dst = static_cast<f16*>(a.out) + row * D + col;
#pragma unroll
          for (int j = 0; j < NB; j += 4)
            *reinterpret_cast<f16x4*>(dst + j) = f16x4{static_cast<f16>(y[j]), static_cast<f16>(y[j + 1]),
                                                       static_cast<f16>(y[j + 2]), static_cast<f16>(y[j + 3])};
        } else {
          float* dst = a.rec_o + (static_cast<int64_t>(rec) * a.rec_rows + g) * D + col;
#pragma unroll
          for (int j = 0; j < NB; j += 4)
            *reinterpret_cast<f32x4*>(dst + j) = f32x4{y[j], y[j + 1], y[j + 2], y[j + 3]};
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = 16 * nb + 4 * jq;
        const f32x4 y = o[nb] * inv;
        if (whole) {
          const f16x4 h = {static_cast<f16>(y[0]), static_cast<f16>(y[1]), static_cast<f16>(y[2]),
                           static_cast<f16>(y[3])};
          *reinterpret_cast<f16x4*>(static_cast<f16*>(a.out) + row * D + col) = h;
        } else {
          *reinterpret_cast<f32x4*>(a.rec_o + (static_cast<int64_t>(rec) * a.rec_rows + g) * D + col) = y;
        }
      }
    }
    if (!whole && jq == 0) {
      a.rec_m[rec * a.rec_rows + g] = piece_bad ? qnan : m;
      a.rec_l[rec * a.rec_rows + g] = piece_bad ? qnan : lt;
    }
  };

  f16x8 kop[KB];
  f16x4 vop[NB];
  bool fbad[NST];
  // E4M3 append mode: this lane's addresses in a stage's new-row area
  const uint32_t nk_addr = ring + static_cast<uint32_t>(16 * jq * KB);
  const uint32_t nv_addr = ring + static_cast<uint32_t>(2 * NB * g);
  auto process = [&](int i, auto stc) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    if (i == 0 || wk.piece_starts(cc)) piece_start(stc, i == 0 || cc.t == 0);
    piece_bad |= fbad[st];
    if constexpr (F8NEW) {
      if (cc.t == cc.nt - 1) {  // the segment's last tile holds the new token, row rn
        // the operands of row rn become the values of the codes the reduce kernel stores
        // for it: code(x * 1/scale), expanded exactly, as for every other row
        const int tn = tau(cc.ctx - 1 - cc.t * TK);  // its product row (tau is an involution)
        u32x4 nkr[KB], nvr;
        read_new_rows_f8<D, st * STAGE + NEWOFF>(nk_addr, nv_addr, nkr, nvr);
        if (g == tn) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            kop[kb] = e4m3_values8(nkr[kb], a.k_sc);
          }
        }
        if (jq == (tn >> 2)) {
          const int t = tn & 3;
          const f16x8 qv = e4m3_values8(nvr, a.v_sc);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const f16 val = qv[nb];
            f16x4 x = vop[nb];
            x[0] = t == 0 ? val : x[0];
            x[1] = t == 1 ? val : x[1];
            x[2] = t == 2 ? val : x[2];
            x[3] = t == 3 ? val : x[3];
            vop[nb] = x;
          }
        }
      }
    }
    consume(min(TK, cc.ctx - cc.t * TK), kop, vop);
    if (i == n_my - 1 || wk.piece_ends(cc)) piece_end();
    wk.advance(cc);
  };

  // ---- main loop, unrolled by the ring depth so that stage offsets are immediates: the
  // fetch cursor runs NST - 1 tiles ahead; every step issues the same K/V loads.  The
  // table entries of the fetch cursor's tile are always loaded one step ahead.
  // Prologue: the cursors of the first NST tiles, and their table entries.  For rings of
  // two and three, all the entries come in one batch of scalar loads (one wait).
  Cursor cf = cc;
  const int32_t *e0, *e1;
  int32_t pe0 = 0, pe1 = 0;
  if constexpr (DENSE) {  // no entries: the first NST - 1 tiles straight away
    unroll<NST - 1>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      fbad[j] = fetch(cf, j < n_my, j < n_my && (j == 0 || cf.t == 0), j, 0, 0);
      wk.advance(cf);
    });
  } else if constexpr (NST == 2) {
    Cursor c1 = cf;
    wk.advance(c1);
    const int32_t *a0, *a1;
    entry_ptrs(cf, true, a0, a1);
    entry_ptrs(c1, 1 < n_my, e0, e1);
    int32_t p[4];
    load_entries4(uniform_ptr(a0), uniform_ptr(a1), uniform_ptr(e0), uniform_ptr(e1), p);
    fbad[0] = fetch(cf, true, true, 0, p[0], p[1]);
    cf = c1;
    pe0 = p[2];
    pe1 = p[3];
  } else if constexpr (NST == 3) {
    Cursor c1 = cf;
    wk.advance(c1);
    Cursor c2 = c1;
    wk.advance(c2);
    const int32_t *a0, *a1, *b0, *b1;
    entry_ptrs(cf, 0 < n_my, a0, a1);
    entry_ptrs(c1, 1 < n_my, b0, b1);
    entry_ptrs(c2, 2 < n_my, e0, e1);
    int32_t p[6];
    load_entries6(uniform_ptr(a0), uniform_ptr(a1), uniform_ptr(b0), uniform_ptr(b1), uniform_ptr(e0),
                  uniform_ptr(e1), p);
    fbad[0] = fetch(cf, 0 < n_my, 0 < n_my, 0, p[0], p[1]);
    fbad[1] = fetch(c1, 1 < n_my, 1 < n_my && c1.t == 0, 1, p[2], p[3]);
    cf = c2;
    pe0 = p[4];
    pe1 = p[5];
  } else {
    unroll<NST - 1>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      const int32_t *a0, *a1;
      entry_ptrs(cf, j < n_my, a0, a1);
      const int32_t p0 = scalar_load(a0), p1 = scalar_load(a1);
      fbad[j] = fetch(cf, j < n_my, j < n_my && (j == 0 || cf.t == 0), j, p0, p1);
      wk.advance(cf);
    });
    entry_ptrs(cf, NST - 1 < n_my, e0, e1);
    pe0 = scalar_load(e0);
    pe1 = scalar_load(e1);
  }
  for (int i0 = 0; i0 < n_my; i0 += NST) {
    unroll<NST>([&](auto stc) __attribute__((always_inline)) {
      constexpr int st = decltype(stc)::value;
      constexpr int nxt = (st + NST - 1) % NST;  // the stage the previous tile was read from
      const int i = i0 + st;
      const bool real = i + NST - 1 < n_my;
      fbad[nxt] = fetch(cf, real, real && cf.t == 0, nxt, pe0, pe1);
      wk.advance(cf);
      if constexpr (DENSE) {
        if constexpr (D == 128) read_stage_d128_dense<VM, st * STAGE>(ka, va, kop, vop);
        else read_stage_d64_dense<VM, st * STAGE>(ka, va, kop, vop);
      } else {
        entry_ptrs(cf, i + NST < n_my, e0, e1);
        if constexpr (F8) read_stage_f8<D, VM, st * STAGE>(ka, va, kop, vop, e0, e1, pe0, pe1);
        else read_stage_mf<D, VM, st * STAGE>(ka, va, kop, vop, e0, e1, pe0, pe1);
      }
      if (i < n_my) process(i, stc);
    });
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load still writes LDS at exit
}

// ---------------------------------------------------------------------------
// decode with shared prefixes (pa_decode_shared): groups of sequences whose tables hold the
// same physical blocks for their first L tokens (parallel samples of one prompt, requests
// that share a cached prefix; [SOSP] section 2.4 and [CON] section 4.3 share such blocks by
// reference counts).  The batch becomes a list of virtual sequences: first each group's
// prefix, whose query rows are the query heads of all its members (at most kShRows per kv
// head), then each sequence's own part, positions L .. ctx - 1.  A prefix is streamed once
// for all its members; every piece goes to a record, and the reduce merges, per query row,
// the pieces of its group's prefix and then those of its own part, in token order.
// ---------------------------------------------------------------------------

struct SharedArgs {
  const int32_t* seq_group;     // [S] the group whose prefix sequence s shares, -1: none
  const int32_t* group_first;   // [NG] first member (the members are consecutive sequences)
  const int32_t* group_size;    // [NG] members
  const int32_t* group_prefix;  // [NG] shared tokens L
  int num_groups;
};

constexpr int kShRows = 32;         // query rows of a prefix per kv head: two 16-row blocks
constexpr int kShWavesPerCU = 3;    // its 16 KB stages (q area doubled) fit three rings per CU

// Whether group gi describes a prefix the kernels can stream: L whole tiles and whole blocks,
// at most max_ctx, 1 .. kShRows / group members that are sequences of the batch.
__device__ __forceinline__ bool shared_group_ok(int L, int n, int f, int S, int group, int bsz, int max_ctx) {
  return L > 0 && L <= max_ctx && L % 16 == 0 && L % bsz == 0 && n >= 1 && n * group <= kShRows && f >= 0 &&
         f <= S - n;
}

// Position of a wave in the list of virtual sequences (all wave-uniform).
struct VCursor {
  int v;       // virtual sequence: group v's prefix (v < NG), else sequence v - NG's own part
  int unit;    // kv head
  int t, nt;   // tile within the segment, tiles in it
  int ctx;     // tokens of the virtual sequence
  int gstart;  // global index of the segment's first tile
  int trow;    // block-table row it reads
  int pos0;    // position of its first token in that row
  int s0;      // sequence of its first query row
  int rows;    // query rows per kv head (members x group, or group)
  int wt;      // cost of one of its tiles
  int c0;      // cost position where the segment starts
};

// The work split.  Waves take equal shares of an estimated cost, not of tiles: a tile of
// one 16-row block costs kShTileCost, one of two blocks kShTileCost2, and each segment
// kShSegCost besides (its start and end: q rows, records, cursor), in units of about
// 0.2 us measured on MI355X.  With equal tile shares, the waves that took many short own
// parts finished last, a piece boundary costing about as much as a tile.  Segment k starts
// at cost position c0 and its tile t sits at c0 + kShSegCost + t wt; wave w takes the tiles
// at positions p with floor(p Wp / total) = w, a contiguous range.  Wp = min(waves,
// total / kShTileCost2), so that every share is at least one tile's cost wide: no wave
// inside a segment's span is left without a tile of it, as the reduce's records require.
constexpr int kShTileCost = 4, kShTileCost2 = 5, kShSegCost = 6;

template <int TK>
struct VWork {
  static constexpr int kChunks = 4;  // chunks of 64 virtual sequences the scans keep per lane
  const int32_t* ctxs;
  SharedArgs sh;
  int S, NG, V, max_ctx, n_units, G, bsz;
  int Wp;         // waves sharing the work
  int total;      // total cost (the host bounds it below 2^31)
  double inv_total;
  int A, n_my;

  // floor(n / d) for 0 <= n < 2^53 and 0 < d < 2^31: a double estimate (off by at most one
  // for these sizes), corrected with exact integer products
  __device__ static int64_t div_floor(int64_t n, int64_t d, double inv_d) {
    int64_t q = static_cast<int64_t>(static_cast<double>(n) * inv_d);
    if (q * d > n) --q;
    else if ((q + 1) * d <= n) ++q;
    return q;
  }

  __device__ static int tiles(int c) { return c > 0 ? (c + TK - 1) / TK : 0; }
  __device__ static int tile_cost(int rows) { return rows > kMfRows ? kShTileCost2 : kShTileCost; }

  // Virtual sequence v: its tokens, table row, first position, first query sequence and
  // query rows per kv head, read with scalar loads (batched: one wait for a prefix, two for
  // an own part).  Tokens are 0 (nothing streamed) for an invalid group, a prefix of no
  // valid group, or an own part that is invalid; the reduce gives the affected rows NaN.
  __device__ void geom(int v, int& ctxv, int& trow, int& pos0, int& s0, int& rows) const {
    // the group's prefix, size and first member (read twice: a batch of four)
    auto group = [&](int gi, int& L, int& n, int& f) __attribute__((always_inline)) {
      int32_t p[4];
      load_entries4(uniform_ptr(sh.group_prefix + gi), uniform_ptr(sh.group_size + gi),
                    uniform_ptr(sh.group_first + gi), uniform_ptr(sh.group_first + gi), p);
      L = p[0];
      n = p[1];
      f = p[2];
    };
    if (v < NG) {
      int L, n, f;
      group(v, L, n, f);
      const bool ok = shared_group_ok(L, n, f, S, G, bsz, max_ctx);
      ctxv = ok ? L : 0;
      trow = ok ? f : 0;
      pos0 = 0;
      s0 = trow;
      rows = ok ? n * G : G;
    } else {
      const int s = v - NG;
      int32_t q[2];
      load_entries2(uniform_ptr(ctxs + s), uniform_ptr(sh.seq_group + s), q);
      const int c = q[0], gi = q[1];
      int L = 0;
      bool ok = c > 0 && c <= max_ctx;
      if (gi >= 0) {
        ok = ok && gi < NG;
        if (ok) {  // the group arrays are read only at valid indexes (they may be empty)
          int n, f;
          group(gi, L, n, f);
          ok = shared_group_ok(L, n, f, S, G, bsz, max_ctx) && s >= f && s < f + n && L <= c;
        }
      }
      ctxv = ok ? c - L : 0;
      trow = s;
      pos0 = ok ? L : 0;
      s0 = s;
      rows = G;
    }
  }

  // The same for the lanes' virtual sequences v (v >= V gives 0 tokens), as vector loads
  // issued at clamped valid indexes whatever the lane's case, in two dependent rounds (the
  // own part's group comes from its sequence), so that the loads of several chunks can be
  // in flight together.  S > 0.
  __device__ void geom_lanes1(int v, int& c, int& gi, int& Lp, int& np, int& fp) const {
    const int s = min(max(v - NG, 0), S - 1);
    c = ctxs[s];
    gi = sh.seq_group[s];
    Lp = np = fp = 0;
    if (NG > 0) {
      const int gv = min(v, NG - 1);
      Lp = sh.group_prefix[gv];
      np = sh.group_size[gv];
      fp = sh.group_first[gv];
    }
  }
  __device__ void geom_lanes2(int v, int c, int gi, int Lp, int np, int fp, int& ctxv, int& trow, int& pos0,
                              int& s0, int& rows) const {
    int Lo = 0, no = 0, fo = 0;
    const bool has_g = v >= NG && gi >= 0 && gi < NG;
    if (NG > 0) {
      const int gc = has_g ? gi : 0;
      Lo = sh.group_prefix[gc];
      no = sh.group_size[gc];
      fo = sh.group_first[gc];
    }
    if (v < NG) {
      const bool ok = shared_group_ok(Lp, np, fp, S, G, bsz, max_ctx);
      ctxv = ok ? Lp : 0;
      trow = ok ? fp : 0;
      pos0 = 0;
      s0 = trow;
      rows = ok ? np * G : G;
    } else {
      const int s = v - NG;
      bool ok = c > 0 && c <= max_ctx;
      if (gi >= 0)
        ok = ok && has_g && shared_group_ok(Lo, no, fo, S, G, bsz, max_ctx) && s >= fo && s < fo + no && Lo <= c;
      const int L = gi >= 0 ? Lo : 0;
      ctxv = ok ? c - L : 0;
      trow = s;
      pos0 = ok ? L : 0;
      s0 = s;
      rows = G;
    }
    if (v >= V) ctxv = 0;
  }

  // Split the work and place cursor c at this wave's first tile (n_my = 0: nothing to do).
  __device__ void init(const StreamArgs& a, const SharedArgs& shv, int w, int lane, int bs, VCursor& c) {
    ctxs = a.context_lens;
    sh = shv;
    S = a.num_seqs;
    NG = sh.num_groups;
    V = NG + S;
    max_ctx = a.max_context_len;
    n_units = a.num_kv_heads;
    G = a.group;
    bsz = bs;
    n_my = 0;
    A = 0;
    const int nch = (V + kWave - 1) / kWave;
    const bool cached = nch <= kChunks;
    int k_ctx[kChunks] = {}, k_trow[kChunks] = {}, k_pos0[kChunks] = {}, k_s0[kChunks] = {}, k_rows[kChunks] = {};
    auto chunk = [&](int b, int& ctxv, int& trow, int& pos0, int& s0, int& rows) __attribute__((always_inline)) {
      int cv, gi, Lp, np, fp;
      geom_lanes1(b * kWave + lane, cv, gi, Lp, np, fp);
      geom_lanes2(b * kWave + lane, cv, gi, Lp, np, fp, ctxv, trow, pos0, s0, rows);
    };
    if (cached) {  // both rounds of loads of all chunks at once
      int cv[kChunks] = {}, gi[kChunks] = {}, Lp[kChunks] = {}, np[kChunks] = {}, fp[kChunks] = {};
#pragma unroll
      for (int b = 0; b < kChunks; ++b)
        if (b < nch) geom_lanes1(b * kWave + lane, cv[b], gi[b], Lp[b], np[b], fp[b]);
#pragma unroll
      for (int b = 0; b < kChunks; ++b)
        if (b < nch)
          geom_lanes2(b * kWave + lane, cv[b], gi[b], Lp[b], np[b], fp[b], k_ctx[b], k_trow[b], k_pos0[b], k_s0[b],
                      k_rows[b]);
    }
    // totals
    int part_tiles = 0, part_cost = 0;
    for (int b = 0; b < nch; ++b) {
      int ctxv, trow, pos0, s0, rows;
      if (cached) {
        ctxv = pick(k_ctx, b);
        rows = pick(k_rows, b);
      } else {
        chunk(b, ctxv, trow, pos0, s0, rows);
      }
      const int nt = tiles(ctxv);
      part_tiles += nt * n_units;
      part_cost += nt > 0 ? n_units * (kShSegCost + nt * tile_cost(rows)) : 0;
    }
    const int T = wave_sum_int(part_tiles);
    total = wave_sum_int(part_cost);
    Wp = min(a.num_waves, total / kShTileCost2);
    if (T == 0 || w >= Wp) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      return;
    }
    inv_total = 1.0 / static_cast<double>(total);
    const double inv_wp = 1.0 / static_cast<double>(Wp);
    const int th0 = static_cast<int>(div_floor(static_cast<int64_t>(w) * total + Wp - 1, Wp, inv_wp));
    const int th1 =
        w + 1 == Wp ? total : static_cast<int>(div_floor(static_cast<int64_t>(w + 1) * total + Wp - 1, Wp, inv_wp));
    // the first tiles at positions >= th0 and >= th1
    int x0 = -1, x1 = T;
    int base_t = 0, base_c = 0;
    for (int b = 0; b < nch && x1 == T; ++b) {
      int ctxv, trow, pos0, s0, rows;
      if (cached) {
        ctxv = pick(k_ctx, b);
        trow = pick(k_trow, b);
        pos0 = pick(k_pos0, b);
        s0 = pick(k_s0, b);
        rows = pick(k_rows, b);
      } else {
        chunk(b, ctxv, trow, pos0, s0, rows);
      }
      const int nt = tiles(ctxv), wt = tile_cost(rows);
      const int tl = nt * n_units, cost = nt > 0 ? n_units * (kShSegCost + nt * wt) : 0;
      const int ti = wave_incl_scan_int(tl), ci = wave_incl_scan_int(cost);
      const int Gv = base_t + ti - tl, Cv = base_c + ci - cost;
      // v's last tile sits at Cv + cost - wt; the first v whose last tile reaches th holds it
      auto find = [&](int th, int& x, bool cursor) __attribute__((always_inline)) {
        const uint64_t hit = __builtin_amdgcn_ballot_w64(nt > 0 && Cv + cost - wt >= th);
        if (hit == 0) return;
        const int l = __builtin_ctzll(hit);
        const int ntl = __builtin_amdgcn_readlane(nt, l), wtl = __builtin_amdgcn_readlane(wt, l);
        const int Cl = __builtin_amdgcn_readlane(Cv, l), Gl = __builtin_amdgcn_readlane(Gv, l);
        const int sz = kShSegCost + ntl * wtl;
        const int rem = th - Cl - kShSegCost - (ntl - 1) * wtl;  // unit u's last tile reaches th
        const int u = rem > 0 ? (rem + sz - 1) / sz : 0;
        const int cs = Cl + u * sz;
        const int rt = th - cs - kShSegCost;
        const int t = rt > 0 ? (rt + wtl - 1) / wtl : 0;
        x = Gl + u * ntl + t;
        if (cursor) {
          c.v = b * kWave + l;
          c.unit = u;
          c.t = t;
          c.nt = ntl;
          c.ctx = __builtin_amdgcn_readlane(ctxv, l);
          c.gstart = Gl + u * ntl;
          c.trow = __builtin_amdgcn_readlane(trow, l);
          c.pos0 = __builtin_amdgcn_readlane(pos0, l);
          c.s0 = __builtin_amdgcn_readlane(s0, l);
          c.rows = __builtin_amdgcn_readlane(rows, l);
          c.wt = wtl;
          c.c0 = cs;
        }
      };
      if (x0 < 0) find(th0, x0, true);
      if (w + 1 < Wp) find(th1, x1, false);
      base_t += __builtin_amdgcn_readlane(ti, kWave - 1);
      base_c += __builtin_amdgcn_readlane(ci, kWave - 1);
    }
    A = x0;
    n_my = x0 < 0 ? 0 : x1 - x0;
    // every load of the scans is complete before the stream's first loads (without this the
    // compiler may drain all of them, the stream's too, in front of the loop)
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  __device__ static int pick(const int (&k)[kChunks], int b) {
    int r = k[0];
#pragma unroll
    for (int i = 1; i < kChunks; ++i) r = b == i ? k[i] : r;
    return r;
  }

  // the wave holding the last tile of c's segment
  __device__ int wave_of_last(const VCursor& c) const {
    const int p = c.c0 + kShSegCost + (c.nt - 1) * c.wt;
    return static_cast<int>(div_floor(static_cast<int64_t>(p) * Wp, total, inv_total));
  }

  __device__ void set(VCursor& c, int v) const {
    c.v = v;
    geom(v, c.ctx, c.trow, c.pos0, c.s0, c.rows);
    c.nt = tiles(c.ctx);
    c.wt = tile_cost(c.rows);
  }

  __device__ void advance(VCursor& c) const {
    if (++c.t < c.nt) return;
    c.c0 += kShSegCost + c.nt * c.wt;
    c.gstart += c.nt;
    c.t = 0;
    if (++c.unit < n_units) return;
    c.unit = 0;
    do {
      if (c.v + 1 >= V) {
        c.v = V;
        c.nt = 0;
        c.ctx = 0;
        break;
      }
      set(c, c.v + 1);
    } while (c.nt == 0);
  }
};

// The shared-prefix stream kernel: the fp16 MFMA stream kernel (3-stage ring, persistent
// waves, equal shares of the estimated cost, VWork) over the virtual sequences, with up to
// two 16-row blocks of query rows per unit (NRB) and every piece written to a record.
template <int D>
__global__ __launch_bounds__(kWave) void pa_shared_mfma_kernel(const StreamArgs a, const SharedArgs sh) {
  using K = MCfg<D, false>;
  constexpr int NST = kMfStages;
  constexpr int TK = K::kTK, KB = K::kKB, NB = K::kNB, NC = K::kNC, ROW = K::kRow;
  constexpr int ROWQ = K::kRowQ, NCQ = K::kNCQ;
  constexpr int LOADS = K::kLoads, HALF = K::kHalf;
  constexpr int NRB = kShRows / kMfRows;        // row blocks per unit
  constexpr int STAGE = 2 * HALF + kShRows * ROWQ;
  constexpr int QOFF = 2 * HALF;
  constexpr int QROWS = 1024 / ROWQ;
  constexpr int VM = (NST - 1) * 2 * LOADS;
  static_assert(VM <= 63, "vmcnt range");
  static_assert(NST * STAGE <= 65536, "stage offsets are 16-bit immediates");
  __shared__ __align__(1024) char s_ring[NST * STAGE];

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int g = lane % 16;
  const int jq = lane / 16;
  const int bsz = a.block_size;

  VWork<TK> wk;
  VCursor cc;
  wk.init(a, sh, w, lane, bsz, cc);
  const int n_my = wk.n_my;
  if (n_my == 0) return;
  const int A = wk.A, A_end = A + n_my;

  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s_ring));
  uint32_t ka[KB], va[NB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int c = jq * KB + kb;
    ka[kb] = ring + static_cast<uint32_t>(g * ROW + ((c ^ swz16<D>(g)) * 16));
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 4 * jq + (g >> 2), q = g & 3;
    const int c = 2 * nb + (q >> 1);
    va[nb] = ring + static_cast<uint32_t>(HALF + r * ROW + ((c ^ swz16<D>(r)) * 16) + (q & 1) * 8);
  }
  const uint32_t qa = ring + static_cast<uint32_t>(g * ROWQ + jq * KB * 16);  // block rb: + 16 rb ROWQ
  uint32_t lo[LOADS];
  bool hi8[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = i * 64 + lane;
    const int r = pos / NC, p = pos % NC;
    const int rr = bsz >= TK ? r : (r & (bsz - 1));
    lo[i] = static_cast<uint32_t>(rr * ROW + ((p ^ swz16<D>(r)) * 16));
    hi8[i] = r >= 8;
  }

  const char* kcache = static_cast<const char*>(a.k_cache);
  const char* vcache = static_cast<const char*>(a.v_cache);
  const char* qbytes = static_cast<const char*>(a.q);
  const uint64_t head_bytes = static_cast<uint64_t>(bsz) * ROW;
  const uint64_t block_bytes = head_bytes * static_cast<uint64_t>(a.num_kv_heads);
  const int G = a.group;

  // table entries of tile f: its first row slot's and, for block size 8, the second half's
  auto entry_ptrs = [&](const VCursor& f, bool real, const int32_t*& e0, const int32_t*& e1)
      __attribute__((always_inline)) {
    if (!real) {
      e0 = e1 = uniform_ptr(a.block_tables);
      return;
    }
    const int tok0 = f.t * TK;
    const int32_t* p = a.block_tables + static_cast<int64_t>(f.trow) * a.max_blocks_per_seq +
                       ((f.pos0 + tok0) >> a.log2_block);
    e0 = uniform_ptr(p);
    e1 = (bsz < TK && tok0 + bsz < f.ctx) ? uniform_ptr(p + 1) : e0;
  };

  auto fetch = [&](const VCursor& f, bool real, bool qload, int st, int p0, int p1)
      __attribute__((always_inline)) -> bool {
    bool bad = false;
    const int kvh = real ? f.unit : 0;
    const int tok0 = f.t * TK;
    if (real) {
      if (p0 < 0 || p0 >= a.num_blocks) {
        bad = true;
        p0 = 0;
      }
      if (bsz < TK && tok0 + bsz < f.ctx) {
        if (p1 < 0 || p1 >= a.num_blocks) {
          bad = true;
          p1 = 0;
        }
      } else {
        p1 = 0;
      }
    } else {
      p0 = 0;
      p1 = 0;
    }
    char* stage = s_ring + st * STAGE;
    if (qload) {  // rows r < f.rows: member r / G's query head kvh G + r % G
#pragma unroll
      for (int i = 0; i < kShRows / QROWS; ++i) {
        if (i * QROWS < f.rows) {
          const int r = min(i * QROWS + lane / NCQ, f.rows - 1);
          const int64_t qrow = static_cast<int64_t>(f.s0 + r / G) * a.num_q_heads + kvh * G + r % G;
          __builtin_amdgcn_global_load_lds(qbytes + qrow * ROWQ + (lane % NCQ) * 16, stage + QOFF + i * 1024, 16, 0,
                                           0);
        }
      }
    }
    const uint64_t head = static_cast<uint64_t>(kvh) * head_bytes;
    const uint64_t b0 = static_cast<uint64_t>(static_cast<uint32_t>(p0)) * block_bytes + head +
                        static_cast<uint64_t>((f.pos0 + tok0) & (bsz - 1)) * ROW * (real ? 1 : 0);
    const uint64_t b1 = static_cast<uint64_t>(static_cast<uint32_t>(p1)) * block_bytes + head;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const bool second = bsz < TK && (K::kRowsPerLoad > 8 ? hi8[i] : i * K::kRowsPerLoad >= 8);
      const uint64_t off = (second ? b1 : b0) + lo[i];
      __builtin_amdgcn_global_load_lds(kcache + off, stage + i * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vcache + off, stage + HALF + i * 1024, 16, 0, 0);
    }
    return bad;
  };

  f16x8 qop[NRB][KB];
  f32x4 o[NRB][NB];
  float m[NRB], l[NRB];
  int rows = 0;
  bool piece_bad = false;

  auto piece_start = [&](auto stc) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    rows = cc.rows;
    unroll<NRB>([&](auto rbc) __attribute__((always_inline)) {
      constexpr int rb = decltype(rbc)::value;
      if (rb == 0 || rows > 16) {
        read_q_mf<KB, st * STAGE + QOFF + rb * 16 * ROWQ>(qa, qop[rb]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qop[rb][kb] = 16 * rb + g < rows ? qop[rb][kb] : f16x8{};
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qop[rb][kb] = f16x8{};
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[rb][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      m[rb] = -INFINITY;
      l[rb] = 0.0f;
    });
    piece_bad = false;
    if (cc.t == 0 && lane == 0)
      a.seg_desc[cc.v * a.n_units + cc.unit] = make_int2(w, wk.wave_of_last(cc));
  };

  auto consume = [&](int cn, const f16x8 (&kop)[KB], f16x4 (&vop)[NB]) __attribute__((always_inline)) {
    constexpr float kRebase = 8.0f;
    const bool full = cn >= TK;
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ok[i] = full || (4 * jq + i < cn);
    if (!full) {  // V rows past the context (poison or block 0) must not reach O
      const uint32_t mlo = (ok[0] ? 0x0000FFFFu : 0u) | (ok[1] ? 0xFFFF0000u : 0u);
      const uint32_t mhi = (ok[2] ? 0x0000FFFFu : 0u) | (ok[3] ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint64_t x = __builtin_bit_cast(uint64_t, vop[nb]);
        x &= (static_cast<uint64_t>(mhi) << 32) | mlo;
        vop[nb] = __builtin_bit_cast(f16x4, x);
      }
    }
    // the score products of every row block first, then each block's softmax and P.V: the
    // second block's products run while the first block's softmax does, and the first
    // block's P.V while the second block's softmax does (matrix and vector instructions of
    // one wave execute together)
    const bool two = rows > 16;  // wave-uniform
    f32x4 scs[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (rb > 0 && !two) break;
      f32x4 sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (kb & 1) sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb], qop[rb][kb], sb, 0, 0, 0);
        else sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb], qop[rb][kb], sa, 0, 0, 0);
      }
      scs[rb] = sa + sb;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (rb > 0 && !two) break;  // wave-uniform: one row block
      const f32x4 sc = scs[rb];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, ok[i] ? sc[i] : -INFINITY);
      {
        const auto x32 = __builtin_amdgcn_permlane32_swap(as_u(mt), as_u(mt), false, false);
        mt = fmaxf(as_f(x32[0]), as_f(x32[1]));
        const auto x16 = __builtin_amdgcn_permlane16_swap(as_u(mt), as_u(mt), false, false);
        mt = fmaxf(as_f(x16[0]), as_f(x16[1]));
      }
      mt *= a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(mt > m[rb] + kRebase) != 0) {
        const float m_new = fmaxf(m[rb], mt);
        const float corr = rescale(m[rb], m_new);
        l[rb] *= corr;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[rb][nb] *= corr;
        m[rb] = m_new;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = ok[i] ? __builtin_amdgcn_exp2f(fmaf(sc[i], a.scale_log2, -m[rb])) : 0.0f;
        l[rb] += p[i];
      }
      const f16x4 pb = {static_cast<f16>(p[0]), static_cast<f16>(p[1]), static_cast<f16>(p[2]),
                        static_cast<f16>(p[3])};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop[nb], pb, o[rb][nb], 0, 0, 0);
    }
  };

  // every piece ends in a record (rows 16 rb + g < rows of each row block): a segment held
  // whole by this wave in the record of its own after the waves' (a share may hold several),
  // a split one in this wave's head or tail record
  auto piece_end = [&]() __attribute__((always_inline)) {
    const bool head = cc.gstart < A;
    const bool whole = !head && cc.gstart + cc.nt <= A_end;
    const int rec = whole ? 2 * a.num_waves + cc.v * a.n_units + cc.unit : w * 2 + (head ? 0 : 1);
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (rb > 0 && rows <= 16) break;
      float lt = l[rb];
      {
        const auto x32 = __builtin_amdgcn_permlane32_swap(as_u(lt), as_u(lt), false, false);
        lt = as_f(x32[0]) + as_f(x32[1]);
        const auto x16 = __builtin_amdgcn_permlane16_swap(as_u(lt), as_u(lt), false, false);
        lt = as_f(x16[0]) + as_f(x16[1]);
      }
      const int row = 16 * rb + g;
      if (row < rows) {
        const float inv = piece_bad ? qnan : 1.0f / lt;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = 16 * nb + 4 * jq;
          const f32x4 y = o[rb][nb] * inv;
          *reinterpret_cast<f32x4*>(a.rec_o + (static_cast<int64_t>(rec) * a.rec_rows + row) * D + col) = y;
        }
        if (jq == 0) {
          a.rec_m[rec * a.rec_rows + row] = piece_bad ? qnan : m[rb];
          a.rec_l[rec * a.rec_rows + row] = piece_bad ? qnan : lt;
        }
      }
    }
  };

  f16x8 kop[KB];
  f16x4 vop[NB];
  bool fbad[NST];
  auto process = [&](int i, auto stc) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    if (i == 0 || cc.t == 0) piece_start(stc);
    piece_bad |= fbad[st];
    consume(min(TK, cc.ctx - cc.t * TK), kop, vop);
    if (i == n_my - 1 || cc.t == cc.nt - 1) piece_end();
    wk.advance(cc);
  };

  VCursor cf = cc;
  const int32_t *e0, *e1;
  int32_t pe0 = 0, pe1 = 0;
  {
    VCursor c1 = cf;
    wk.advance(c1);
    VCursor c2 = c1;
    wk.advance(c2);
    const int32_t *a0, *a1, *b0, *b1;
    entry_ptrs(cf, true, a0, a1);
    entry_ptrs(c1, 1 < n_my, b0, b1);
    entry_ptrs(c2, 2 < n_my, e0, e1);
    int32_t p[6];
    load_entries6(uniform_ptr(a0), uniform_ptr(a1), uniform_ptr(b0), uniform_ptr(b1), uniform_ptr(e0),
                  uniform_ptr(e1), p);
    fbad[0] = fetch(cf, true, true, 0, p[0], p[1]);
    fbad[1] = fetch(c1, 1 < n_my, 1 < n_my && c1.t == 0, 1, p[2], p[3]);
    cf = c2;
    pe0 = p[4];
    pe1 = p[5];
  }
  static_assert(NST == 3, "the prologue fills two stages");
  for (int i0 = 0; i0 < n_my; i0 += NST) {
    unroll<NST>([&](auto stc) __attribute__((always_inline)) {
      constexpr int st = decltype(stc)::value;
      constexpr int nxt = (st + NST - 1) % NST;
      const int i = i0 + st;
      const bool real = i + NST - 1 < n_my;
      fbad[nxt] = fetch(cf, real, real && cf.t == 0, nxt, pe0, pe1);
      wk.advance(cf);
      entry_ptrs(cf, i + NST < n_my, e0, e1);
      read_stage_mf<D, VM, st * STAGE>(ka, va, kop, vop, e0, e1, pe0, pe1);
      if (i < n_my) process(i, stc);
    });
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load still writes LDS at exit
}

// The reduce of pa_decode_shared: one wave per (sequence, query head).  Row (s, h) merges,
// in token order, the pieces of its group's prefix segment (row (s - first) G + h % G of
// those records) and the pieces of its own part (row h % G); zero for an empty context, NaN
// for an invalid one or an invalid group.
template <int D>
__global__ __launch_bounds__(kWave) void pa_shared_reduce_kernel(f16* __restrict__ out, const int2* __restrict__ seg_desc,
                                                                 const float* __restrict__ rec_m,
                                                                 const float* __restrict__ rec_l,
                                                                 const float* __restrict__ rec_o,
                                                                 const int32_t* __restrict__ context_lens,
                                                                 const SharedArgs sh, int num_seqs, int num_q_heads,
                                                                 int group, int n_units, int max_context_len,
                                                                 int block_size, int waves, int rec_rows) {
  constexpr int kDPL = D / kWave;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  f16* dst = out + (static_cast<int64_t>(s) * num_q_heads + h) * D;
  const int kvh = h / group, hg = h - kvh * group;
  const int NG = sh.num_groups;
  // two rounds of loads: the sequence's context, group and own-part descriptor, then the
  // group's arrays and prefix descriptor
  const int ctx = context_lens[s];
  const int gi = sh.seq_group[s];
  const int sp = gi * n_units + kvh, so = (NG + s) * n_units + kvh;
  const int2 dn0 = seg_desc[so];  // read whether or not there is an own part
  bool ok = ctx >= 0 && ctx <= max_context_len;
  int L = 0, f = 0;
  int2 dp = make_int2(0, -1);
  if (gi >= 0) {
    ok = ok && gi < NG;
    if (ok) {  // the group arrays are read only at valid indexes (they may be empty)
      L = sh.group_prefix[gi];
      const int n = sh.group_size[gi];
      f = sh.group_first[gi];
      dp = seg_desc[sp];
      ok = shared_group_ok(L, n, f, num_seqs, group, block_size, max_context_len) && s >= f && s < f + n &&
           L <= ctx;
    }
  }
  if (!ok) {
#pragma unroll
    for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<f16>(__builtin_nanf(""));
    return;
  }
  if (ctx == 0) {
#pragma unroll
    for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<f16>(0.0f);
    return;
  }
  // the two lists of pieces: the prefix segment (group gi, row (s - f) G + hg) and the own
  // segment (sequence s, row hg); a segment held whole by one wave has one piece, in the
  // record 2 waves + its segment index
  const int2 dn = ctx > L ? dn0 : make_int2(0, -1);
  const int np0 = dp.y - dp.x + 1, np1 = dn.y - dn.x + 1;
  const bool desc_ok = (gi < 0 || (dp.x >= 0 && dp.x <= dp.y && dp.y < waves)) &&
                       (ctx <= L || (dn.x >= 0 && dn.x <= dn.y && dn.y < waves));
  if (!desc_ok) {  // not written by the stream kernel
#pragma unroll
    for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<f16>(__builtin_nanf(""));
    return;
  }
  const int rp = (s - f) * group + hg;
  auto idx = [&](int p) {  // flat record row of piece p, in token order
    const bool pre = p < np0;
    const int q = pre ? p : p - np0;
    const int2 d = pre ? dp : dn;
    const int rec = d.x == d.y ? 2 * waves + (pre ? sp : so) : (q == 0 ? d.x * 2 + 1 : (d.x + q) * 2);
    return rec * rec_rows + (pre ? rp : hg);
  };
  merge_indexed<f16, D>(dst, rec_m, rec_l, rec_o, np0 + np1, idx, lane);
}

// ---------------------------------------------------------------------------
// Several query tokens per sequence: causal attention of a prompt chunk over the paged
// cache.  Sequence s has n = query_start[s+1] - query_start[s] query tokens, the last n
// positions of its context; query i (position ctx - n + i) sees positions 0 .. ctx - n + i.
//
// One work-group of four waves per (query-row block, kv head, sequence).  The rows of a
// (sequence, kv head) are its chunk tokens times the G query heads of the group, token
// major; a work-group takes 16 * NR of them per wave (NR 16-row product blocks), and every
// K/V tile it brings into LDS serves all of its rows.  The tiles hold 32 keys and pass
// through an NST-stage ring that the four waves fill together (each loads 8 key rows, which
// lie in one block for block sizes 8, 16 and 32) and read after a barrier.  Per tile and
// 16-row block: scores S^T = K Q^T with two 16x16x32 products per 32 dims (one per key
// half), and O^T += V^T P^T with one 16x16x32 product per 16 dims, its 32 keys in the
// order {4j..4j+3, 16+4j..16+4j+3} of lane quarter j, which is where the two score halves
// leave them; V^T comes from two transposing reads.  Rows past the chunk, keys past a
// row's position and keys past the context are masked; the mask is built only for tiles
// that cross one of those limits.
// ---------------------------------------------------------------------------

// max(a, b, c) in one instruction.  fmaxf would first quieten each operand that is not
// known to be a quiet NaN (the products' outputs are not), one extra instruction per value.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

constexpr int kPfWaves = 4;                            // waves per work-group
constexpr int kPfInterleave = 2;                       // blocks whose score products interleave
constexpr int kPfKeys = 32;                            // keys per tile
constexpr int kPfStages = 2;
constexpr int kPfBlocks = 2;  // 16-row product blocks per wave: 32 query rows

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  float scale_log2;
  int block_size;
  int log2_block;
  int num_kv_heads;
  int num_q_heads;
  int group;
  int max_blocks_per_seq;
  int max_query_len;
  int max_context_len;
  int64_t num_blocks;
  int n_row_blocks;  // work-groups per (sequence, kv head)
  int rb_outer;      // grid (kv head, sequence, row block) instead of (row block, kv head, sequence)
};

template <int D>
struct PCfg {
  static constexpr int kRow = D * 2;                      // bytes per fp16 row
  static constexpr int kNC = kRow / 16;                   // 16-byte chunks per row
  static constexpr int kTile = kPfKeys * kRow;            // bytes of K (or V) per tile
  static constexpr int kStage = 2 * kTile;
  static constexpr int kWaveRows = kPfKeys / kPfWaves;    // key rows each wave loads
  static constexpr int kLoads = kWaveRows * kRow / 1024;  // 1 KB loads per wave for each of K, V
  static constexpr int kKB = D / 32;
  static constexpr int kNB = D / 16;
  static_assert(kLoads * 1024 == kWaveRows * kRow, "a wave loads whole rows");
};

// Stage read of the prefill ring, D = 128: issue the scalar load of the next table entry,
// wait for this wave's loads of the stage, meet the other waves at the barrier (their
// loads have landed and none still reads the stage to be refilled next), then read the K
// operands of both key halves (the second half is 16 rows further), and issue the V^T
// reads without waiting for them: they land while the score products run, and
// pf_wait_v_d128 waits for them before the V operands are used.
template <int VM, int OFF, int ROW>
__device__ __forceinline__ void pf_read_d128(const uint32_t (&ka)[4], const uint32_t (&va)[8],
                                             f16x8 (&k)[2][4], f16x4 (&v)[2][8], const int32_t* e,
                                             int32_t& p) {
  asm volatile(
      "s_load_dword %[p], %[e], 0x0\n\t"
      "s_waitcnt vmcnt(%[vm])\n\t"
      "s_barrier\n\t"
      "ds_read_b128 %[k00], %[ka0] offset:%[o0]\n\t"
      "ds_read_b128 %[k01], %[ka1] offset:%[o0]\n\t"
      "ds_read_b128 %[k02], %[ka2] offset:%[o0]\n\t"
      "ds_read_b128 %[k03], %[ka3] offset:%[o0]\n\t"
      "ds_read_b128 %[k10], %[ka0] offset:%[o1]\n\t"
      "ds_read_b128 %[k11], %[ka1] offset:%[o1]\n\t"
      "ds_read_b128 %[k12], %[ka2] offset:%[o1]\n\t"
      "ds_read_b128 %[k13], %[ka3] offset:%[o1]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k00] "=&v"(k[0][0]), [k01] "=&v"(k[0][1]), [k02] "=&v"(k[0][2]), [k03] "=&v"(k[0][3]),
        [k10] "=&v"(k[1][0]), [k11] "=&v"(k[1][1]), [k12] "=&v"(k[1][2]), [k13] "=&v"(k[1][3]),
        [p] "=&s"(p)
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [ka2] "v"(ka[2]), [ka3] "v"(ka[3]), [e] "s"(e),
        [vm] "n"(VM), [o0] "n"(OFF), [o1] "n"(OFF + 16 * ROW)
      : "memory");
  asm volatile(
      "ds_read_b64_tr_b16 %[v00], %[va0] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v01], %[va1] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v02], %[va2] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v03], %[va3] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v04], %[va4] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v05], %[va5] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v06], %[va6] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v07], %[va7] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v10], %[va0] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v11], %[va1] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v12], %[va2] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v13], %[va3] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v14], %[va4] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v15], %[va5] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v16], %[va6] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v17], %[va7] offset:%[o1]"
      : [v00] "=&v"(v[0][0]), [v01] "=&v"(v[0][1]), [v02] "=&v"(v[0][2]), [v03] "=&v"(v[0][3]),
        [v04] "=&v"(v[0][4]), [v05] "=&v"(v[0][5]), [v06] "=&v"(v[0][6]), [v07] "=&v"(v[0][7]),
        [v10] "=&v"(v[1][0]), [v11] "=&v"(v[1][1]), [v12] "=&v"(v[1][2]), [v13] "=&v"(v[1][3]),
        [v14] "=&v"(v[1][4]), [v15] "=&v"(v[1][5]), [v16] "=&v"(v[1][6]), [v17] "=&v"(v[1][7])
      : [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]), [va4] "v"(va[4]),
        [va5] "v"(va[5]), [va6] "v"(va[6]), [va7] "v"(va[7]), [o0] "n"(OFF), [o1] "n"(OFF + 16 * ROW)
      : "memory");
}

// The V^T reads pf_read_d128 issued have landed: the 16 registers they write are in-out
// operands, so nothing reads them before this wait.  The score accumulators are inputs, so
// that every score product (they need no V) is issued before it; being inputs only, the
// products stay their last writers and the usual wait states before reading them hold.
__device__ __forceinline__ void pf_wait_v_d128(f16x4 (&v)[2][8], const f32x4 (&s)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[0][2]), "+v"(v[0][3]), "+v"(v[0][4]), "+v"(v[0][5]),
                 "+v"(v[0][6]), "+v"(v[0][7]), "+v"(v[1][0]), "+v"(v[1][1]), "+v"(v[1][2]), "+v"(v[1][3]),
                 "+v"(v[1][4]), "+v"(v[1][5]), "+v"(v[1][6]), "+v"(v[1][7])
               : "v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3])
               : "memory");
}

template <int VM, int OFF, int ROW>
__device__ __forceinline__ void pf_read_d64(const uint32_t (&ka)[2], const uint32_t (&va)[4],
                                            f16x8 (&k)[2][2], f16x4 (&v)[2][4], const int32_t* e,
                                            int32_t& p) {
  asm volatile(
      "s_load_dword %[p], %[e], 0x0\n\t"
      "s_waitcnt vmcnt(%[vm])\n\t"
      "s_barrier\n\t"
      "ds_read_b128 %[k00], %[ka0] offset:%[o0]\n\t"
      "ds_read_b128 %[k01], %[ka1] offset:%[o0]\n\t"
      "ds_read_b128 %[k10], %[ka0] offset:%[o1]\n\t"
      "ds_read_b128 %[k11], %[ka1] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v00], %[va0] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v01], %[va1] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v02], %[va2] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v03], %[va3] offset:%[o0]\n\t"
      "ds_read_b64_tr_b16 %[v10], %[va0] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v11], %[va1] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v12], %[va2] offset:%[o1]\n\t"
      "ds_read_b64_tr_b16 %[v13], %[va3] offset:%[o1]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k00] "=&v"(k[0][0]), [k01] "=&v"(k[0][1]), [k10] "=&v"(k[1][0]), [k11] "=&v"(k[1][1]),
        [v00] "=&v"(v[0][0]), [v01] "=&v"(v[0][1]), [v02] "=&v"(v[0][2]), [v03] "=&v"(v[0][3]),
        [v10] "=&v"(v[1][0]), [v11] "=&v"(v[1][1]), [v12] "=&v"(v[1][2]), [v13] "=&v"(v[1][3]),
        [p] "=&s"(p)
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]),
        [va3] "v"(va[3]), [e] "s"(e), [vm] "n"(VM), [o0] "n"(OFF), [o1] "n"(OFF + 16 * ROW)
      : "memory");
}

// NR 16-row product blocks per wave, an NST-stage ring
template <int D, int NR, int NST>
__global__ __launch_bounds__(kPfWaves * kWave, 2) void pa_prefill_kernel(const PrefillArgs a) {
  using C = PCfg<D>;
  constexpr int ROW = C::kRow, NC = C::kNC, TILE = C::kTile, STAGE = C::kStage;
  constexpr int LOADS = C::kLoads, KB = C::kKB, NB = C::kNB;
  constexpr int kPfRows = kPfWaves * NR * 16;  // query rows per work-group
  constexpr int VM = (NST - 2) * 2 * LOADS;    // loads younger than the stage being read
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  static_assert(NST * STAGE + 16 * ROW <= 65536, "LDS offsets are 16-bit immediates");
  __shared__ __align__(1024) char s_ring[NST * STAGE];
  __shared__ int s_bad;

  // wave in the work-group, known uniform: what depends only on it and the tile (table
  // entries, load bases) is scalar work
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane % 16, jq = lane / 16;
  // work-groups start in grid order as compute units free up; the longest row blocks (the
  // last of each chunk) come first, within each (sequence, kv head) or, with rb_outer, over
  // the whole grid
  const int rb = a.n_row_blocks - 1 - static_cast<int>(a.rb_outer ? blockIdx.z : blockIdx.x);
  const int kvh = a.rb_outer ? blockIdx.x : blockIdx.y;
  const int s = a.rb_outer ? blockIdx.y : blockIdx.z;
  const int G = a.group;

  // every value below is uniform over the work-group
  const int r0 = a.query_start[s];
  const int n = a.query_start[s + 1] - r0;
  const int ctx = a.context_lens[s];
  const int row_lo = rb * kPfRows;  // first row (token-major: token * G + head)
  if (n <= 0 || row_lo >= n * G) return;
  const int row_hi = min(n * G, row_lo + kPfRows);  // one past the last row
  const int t_last = (row_hi - 1) / G;
  f16* out = static_cast<f16*>(a.out);
  const int64_t hq = a.num_q_heads;
  auto out_row = [&](int t, int hg) { return out + ((static_cast<int64_t>(r0) + t) * hq + kvh * G + hg) * D; };

  if (n > ctx || ctx > a.max_context_len || n > a.max_query_len) {  // invalid: NaN rows
    for (int r = row_lo + static_cast<int>(threadIdx.x) / (D / 8); r < row_hi; r += kPfWaves * kWave / (D / 8))
      *reinterpret_cast<u32x4*>(out_row(r / G, r % G) + (threadIdx.x % (D / 8)) * 8) =
          u32x4{0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u};
    return;
  }
  const int kend = ctx - n + t_last + 1;  // keys the work-group needs: 0 .. kend - 1 (<= ctx)
  const int T = (kend + kPfKeys - 1) / kPfKeys;

  // ---- query rows of this lane: row 16 NR w + 16 nr + g of the block; its position limit
  int lim[NR];
  bool rvalid[NR];
  f16x8 qop[NR][KB];
  int wave_min_lim = 0x7FFFFFFF;
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    const int r = row_lo + 16 * NR * w + 16 * nr + g;
    rvalid[nr] = r < row_hi;
    const int t = r / G;
    lim[nr] = rvalid[nr] ? ctx - n + t : kend - 1;  // last key the row sees
    const f16* qr = static_cast<const f16*>(a.q) + ((static_cast<int64_t>(r0) + t) * hq + kvh * G + r % G) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qop[nr][kb] = rvalid[nr] ? *reinterpret_cast<const f16x8*>(qr + (jq * KB + kb) * 8) : f16x8{};
  }
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) wave_min_lim = min(wave_min_lim, lim[nr]);
  wave_min_lim = wave_min_int(wave_min_lim);

  // ---- LDS addresses of the operands (first key half; the second is 16 rows further)
  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s_ring));
  uint32_t ka[KB], va[NB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    ka[kb] = ring + static_cast<uint32_t>(g * ROW + (((jq * KB + kb) ^ swz16<D>(g)) * 16));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 4 * jq + (g >> 2), qq = g & 3;
    const int c = 2 * nb + (qq >> 1);
    va[nb] = ring + static_cast<uint32_t>(TILE + r * ROW + ((c ^ swz16<D>(r)) * 16) + (qq & 1) * 8);
  }
  // loads: wave w brings key rows 8 w .. 8 w + 7 of each tile; load i, lane l fills LDS
  // position 64 i + l of that run (row rr, chunk position p, holding chunk p ^ swz16(row))
  uint32_t lo[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = i * 64 + lane;
    const int rr = pos / NC, pp = pos % NC;
    lo[i] = static_cast<uint32_t>(rr * ROW + ((pp ^ swz16<D>((C::kWaveRows * w + rr) & 15)) * 16));
  }
  const int bsz = a.block_size;
  const uint64_t head_bytes = static_cast<uint64_t>(bsz) * ROW;
  const uint64_t block_bytes = head_bytes * static_cast<uint64_t>(a.num_kv_heads);
  const char* kcache = static_cast<const char*>(a.k_cache);
  const char* vcache = static_cast<const char*>(a.v_cache);
  const int32_t* trow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;

  // table entry of this wave's rows in tile f (a valid address for phantom tiles)
  auto entry_ptr = [&](int f) __attribute__((always_inline)) -> const int32_t* {
    const int key0 = f * kPfKeys + C::kWaveRows * w;
    return uniform_ptr(key0 < kend ? trow + (key0 >> a.log2_block) : a.block_tables);
  };
  int bad = 0;  // uniform: a table entry of this wave's rows lay outside the pool
  auto fetch = [&](int f, int st, int p) __attribute__((always_inline)) {
    const int key0 = f * kPfKeys + C::kWaveRows * w;
    const bool real = key0 < kend;  // phantom tiles and rows past the context read block 0
    p = __builtin_amdgcn_readfirstlane(p);  // a scalar load's result: uniform
    const bool outside = real && (p < 0 || p >= a.num_blocks);
    bad |= outside ? 1 : 0;
    if (outside || !real) p = 0;
    const uint64_t base = static_cast<uint64_t>(static_cast<uint32_t>(p)) * block_bytes +
                          static_cast<uint64_t>(kvh) * head_bytes +
                          static_cast<uint64_t>(real ? (key0 & (bsz - 1)) : 0) * ROW;
    char* dst = s_ring + st * STAGE + C::kWaveRows * w * ROW;
    const char* kb = uniform_ptr(kcache + base);  // scalar bases, 32-bit per-lane offsets
    const char* vb = uniform_ptr(vcache + base);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      // (explicit casts: without them the host pass of this compiler drops the kernel)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + lo[i]), static_cast<void*>(dst + i * 1024), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vb + lo[i]),
                                       static_cast<void*>(dst + TILE + i * 1024), 16, 0, 0);
    }
  };

  // ---- softmax state and accumulators.  The row sums come from the matrix cores as well:
  // ones^T P^T puts sum_k p(q, k) (of the fp16 probabilities the P.V product uses) in every
  // element of lane (q, .), one product per block and tile instead of 8 additions per lane.
  f32x4 o[NR][NB], lsum[NR];
  float m[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    m[nr] = -INFINITY;
    lsum[nr] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nr][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const f16 one = static_cast<f16>(1.0f);
  const f16x8 ones = {one, one, one, one, one, one, one, one};

  // Softmax of block nr over the tile, then its P.V products; unmasked: no key of the tile
  // lies past any row's limit (wave-uniform), so interior tiles skip the masking.  A masked
  // score becomes -inf, whose exp2 is 0: every row sees key 0 (its limit is at least 0), so
  // from the first tile on its reference maximum is finite.
  auto block_pv = [&](auto nrc, int key_base, bool unmasked, const f32x4 (&scr)[2],
                      const f16x4 (&vop)[2][NB]) __attribute__((always_inline)) {
    constexpr int nr = decltype(nrc)::value;
    constexpr float kRebase = 8.0f;
    f32x4 sc[2] = {scr[0], scr[1]};
    if (!unmasked) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[kh][i] = key_base + 16 * kh + 4 * jq + i <= lim[nr] ? sc[kh][i] : -INFINITY;
    }
    float mt = max3f(sc[0][0], sc[0][1], sc[0][2]);
    mt = max3f(mt, sc[0][3], sc[1][0]);
    mt = max3f(mt, sc[1][1], sc[1][2]);
    mt = max3f(mt, sc[1][3], sc[1][3]);
    {
      const auto x32 = __builtin_amdgcn_permlane32_swap(as_u(mt), as_u(mt), false, false);
      mt = max3f(as_f(x32[0]), as_f(x32[1]), as_f(x32[1]));
      const auto x16 = __builtin_amdgcn_permlane16_swap(as_u(mt), as_u(mt), false, false);
      mt = max3f(as_f(x16[0]), as_f(x16[1]), as_f(x16[1]));
    }
    mt *= a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mt > m[nr] + kRebase) != 0) {
      const float m_new = fmaxf(m[nr], mt);
      const float corr = rescale(m[nr], m_new);
      lsum[nr] *= corr;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nr][nb] *= corr;
      m[nr] = m_new;
    }
    float p[2][4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[kh][i] = __builtin_amdgcn_exp2f(fmaf(sc[kh][i], a.scale_log2, -m[nr]));
    const f16x8 pb = {static_cast<f16>(p[0][0]), static_cast<f16>(p[0][1]), static_cast<f16>(p[0][2]),
                      static_cast<f16>(p[0][3]), static_cast<f16>(p[1][0]), static_cast<f16>(p[1][1]),
                      static_cast<f16>(p[1][2]), static_cast<f16>(p[1][3])};
    lsum[nr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb, lsum[nr], 0, 0, 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f16x8 vt = {vop[0][nb][0], vop[0][nb][1], vop[0][nb][2], vop[0][nb][3],
                        vop[1][nb][0], vop[1][nb][1], vop[1][nb][2], vop[1][nb][3]};
      o[nr][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vt, pb, o[nr][nb], 0, 0, 0);
    }
  };

  auto consume = [&](int f, const f16x8 (&kop)[2][KB], f16x4 (&vop)[2][NB]) __attribute__((always_inline)) {
    const int key_base = f * kPfKeys;
    // uniform: no key of the tile lies past any row's limit
    const bool unmasked = key_base + kPfKeys - 1 <= wave_min_lim;
    // blocks in groups of NI: the scores of a group with the dim chunk outermost, so its
    // 2 NI accumulation chains interleave, then each block's softmax and P.V
    constexpr int NI = kPfInterleave < NR ? kPfInterleave : NR;
    static_assert(NR % NI == 0, "whole groups");
    unroll<NR / NI>([&](auto gc) __attribute__((always_inline)) {
      constexpr int g0 = decltype(gc)::value * NI;
      f32x4 sc[NI][2];
#pragma unroll
      for (int b = 0; b < NI; ++b) sc[b][0] = sc[b][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int b = 0; b < NI; ++b)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
            sc[b][kh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kh][kb], qop[g0 + b][kb], sc[b][kh], 0, 0, 0);
      if constexpr (g0 == 0) {
        if constexpr (D == 128) {  // the V^T reads have landed, after the score products
          static_assert(NI == 2, "the wait holds the score chains of two blocks");
          const f32x4 s4[4] = {sc[0][0], sc[0][1], sc[1][0], sc[1][1]};
          pf_wait_v_d128(vop, s4);
        }
        if (key_base + kPfKeys > kend) {  // V rows at or past kend (poison, or block 0) must not reach O
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            uint32_t mlo = 0u, mhi = 0u;
            const int k0 = key_base + 16 * kh + 4 * jq;
            mlo |= (k0 + 0 < kend) ? 0x0000FFFFu : 0u;
            mlo |= (k0 + 1 < kend) ? 0xFFFF0000u : 0u;
            mhi |= (k0 + 2 < kend) ? 0x0000FFFFu : 0u;
            mhi |= (k0 + 3 < kend) ? 0xFFFF0000u : 0u;
            const uint64_t msk = (static_cast<uint64_t>(mhi) << 32) | mlo;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              vop[kh][nb] = __builtin_bit_cast(f16x4, __builtin_bit_cast(uint64_t, vop[kh][nb]) & msk);
          }
        }
      }
      unroll<NI>([&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value;
        block_pv(std::integral_constant<int, g0 + b>{}, key_base, unmasked, sc[b], vop);
      });
    });
  };

  // ---- prologue: the flag, then the first NST - 1 tiles
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if constexpr (NST == 3) {
    int32_t pe[2];
    load_entries2(entry_ptr(0), entry_ptr(1), pe);
    fetch(0, 0, pe[0]);
    fetch(1, 1, pe[1]);
  } else {
    unroll<NST - 1>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      fetch(j, j, scalar_load(entry_ptr(j)));
    });
  }
  f16x8 kop[2][KB];
  f16x4 vop[2][NB];
  for (int i0 = 0; i0 < T; i0 += NST) {
    unroll<NST>([&](auto stc) __attribute__((always_inline)) {
      constexpr int st = decltype(stc)::value;
      constexpr int nxt = (st + NST - 1) % NST;
      const int i = i0 + st;
      if (i >= T) return;
      int32_t pn;
      if constexpr (D == 128) pf_read_d128<VM, st * STAGE, ROW>(ka, va, kop, vop, entry_ptr(i + NST - 1), pn);
      else pf_read_d64<VM, st * STAGE, ROW>(ka, va, kop, vop, entry_ptr(i + NST - 1), pn);
      fetch(i + NST - 1, nxt, pn);
      consume(i, kop, vop);
    });
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load still writes LDS
  if (bad) s_bad = 1;
  __syncthreads();
  const bool any_bad = s_bad != 0;

  // ---- rows: o / l, or NaN when a table entry was outside the pool
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    const float lt = lsum[nr][0];  // the whole row's sum, in every lane of the row
    if (!rvalid[nr]) continue;
    const int r = row_lo + 16 * NR * w + 16 * nr + g;
    const float inv = any_bad ? __builtin_nanf("") : 1.0f / lt;
    f16* dst = out_row(r / G, r % G);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f32x4 y = o[nr][nb] * inv;
      *reinterpret_cast<f16x4*>(dst + 16 * nb + 4 * jq) =
          f16x4{static_cast<f16>(y[0]), static_cast<f16>(y[1]), static_cast<f16>(y[2]), static_cast<f16>(y[3])};
    }
  }
}

// ---------------------------------------------------------------------------
// decode, second launch (of every decode call, or pa_decode_reduce alone): one wave per
// (sequence, query head).  Empty or invalid contexts get their zero or NaN row
// here; a segment held whole by one wave (or of one partition) was written by it; a
// segment split over waves w0..w1 is merged from the tail record of w0 and the head
// records of w0+1..w1, and one cut into fixed partitions from its partitions' records.
// ---------------------------------------------------------------------------

template <typename T, int D, int GT>
__global__ __launch_bounds__(kWave) void pa_reduce_kernel(
    T* __restrict__ out, const int2* __restrict__ seg_desc, const float* __restrict__ rec_m,
    const float* __restrict__ rec_l, const float* __restrict__ rec_o,
    const int32_t* __restrict__ context_lens, int num_q_heads, int group, int n_gtiles,
    int max_context_len, int w_cap, int rec_rows, int parts, int64_t rec_cap, const AppendArgs ap) {
  constexpr int kDPL = D / kWave;  // dims per lane
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  T* dst = out + (static_cast<int64_t>(s) * num_q_heads + h) * D;
  const int kvh = h / group;
  const int gtile = (h - kvh * group) / GT;
  const int g = h - kvh * group - gtile * GT;
  const int n_units = (num_q_heads / group) * n_gtiles;
  const int ctx = context_lens[s];  // both loads in flight together
  const int2 d = seg_desc[s * n_units + kvh * n_gtiles + gtile];
  if (ap.k_new != nullptr && h == kvh * group && ctx >= 1 && ctx <= max_context_len) {
    // append mode: the first query head of each kv head stores the new token's K and V
    // rows at position ctx - 1 (the stream kernel read them from k_new / v_new)
    constexpr int kIn = D * static_cast<int>(sizeof(T));  // bytes of an input row
    static_assert(2 * (kIn / 16) <= kWave, "one lane per 16 bytes of the K and V rows");
    const int64_t blk = ap.block_tables[static_cast<int64_t>(s) * ap.max_blocks_per_seq +
                                        (ctx - 1) / ap.block_size];
    const int64_t row = static_cast<int64_t>(s) * ap.num_kv_heads + kvh;
    const int64_t slot = (blk * ap.num_kv_heads + kvh) * ap.block_size + (ctx - 1) % ap.block_size;
    if (blk >= 0 && blk < ap.num_blocks) {
      if (ap.codes) {  // one lane per 16 codes: two 16-byte chunks of fp16 in, one out
        constexpr int kC = D / 16;
        if (lane < 2 * kC) {
          const int c = lane % kC;
          const bool isv = lane >= kC;
          const char* src = (isv ? ap.v_new : ap.k_new) + row * (2 * D) + c * 32;
          const F8Scale sc = isv ? ap.v_sc : ap.k_sc;
          const u32x2 lo = encode8(*reinterpret_cast<const u32x4*>(src), sc);
          const u32x2 hi = encode8(*reinterpret_cast<const u32x4*>(src + 16), sc);
          *reinterpret_cast<u32x4*>((isv ? ap.v_cache : ap.k_cache) + slot * D + c * 16) =
              u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      } else if (lane < 2 * (kIn / 16)) {  // one lane per 16-byte chunk
        constexpr int kC = kIn / 16;
        const int c = lane % kC;
        const bool isv = lane >= kC;
        *reinterpret_cast<u32x4*>((isv ? ap.v_cache : ap.k_cache) + slot * kIn + c * 16) =
            *reinterpret_cast<const u32x4*>((isv ? ap.v_new : ap.k_new) + row * kIn + c * 16);
      }
    }
  }
  if (ctx <= 0 || ctx > max_context_len) {  // nothing to attend over: zeros; invalid: NaN
    const T fill = static_cast<T>(ctx == 0 ? 0.0f : __builtin_nanf(""));
#pragma unroll
    for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = fill;
    return;
  }
  if (parts) {  // fixed partitions: d = {first partition's record, partitions}
    if (d.y == 1) return;  // one partition: the stream kernel wrote the row
    if (d.x < 0 || d.y < 1 || static_cast<int64_t>(d.x) + d.y > rec_cap) {  // not written by the stream kernel
#pragma unroll
      for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<T>(__builtin_nanf(""));
      return;
    }
    merge_indexed<T, D>(dst, rec_m, rec_l, rec_o, d.y, [&](int p) { return (d.x + p) * rec_rows + g; }, lane);
    return;
  }
  if (d.x == d.y) return;  // one wave held the whole segment and wrote the row
  if (d.x < 0 || d.x > d.y || d.y >= w_cap) {  // not written by the stream kernel: no records
#pragma unroll
    for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<T>(__builtin_nanf(""));
    return;
  }
  merge_row<T, D>(dst, rec_m, rec_l, rec_o, d.x, d.y - d.x + 1, rec_rows, g, lane);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

using pa_detail::fail;
using pa_detail::g_error;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// An E4M3 store scale and its reciprocal, rounded once to fp32 (the kernels use it to find
// the two codes nearest to x / scale, and the scale itself to choose between them exactly)
F8Scale f8_scale(float scale) { return F8Scale{scale, static_cast<float>(1.0 / static_cast<double>(scale))}; }

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

// Query rows per wave: the fp16 kernel's products take 16 (unused ones are zero); the
// fp32 kernel keeps 1, 2, 4 or 8 rows in registers (padded rows are masked).
int group_tile(int group, int dtype) {
  if (dtype == PA_F16) return kMfRows;
  return group >= 5 ? 8 : group >= 3 ? 4 : group;
}

// Geometry shared by the size query, the stream launch and the reduce launch.
struct Geom {
  int gt = 1;        // query heads per unit
  int n_gtiles = 1;  // units per kv head
  int n_units = 1;   // segments per sequence
  int rec_rows = 1;  // query rows per piece record
  int w_cap = 1;     // waves a launch may use (the default split's records are per wave)
  int part = 0;      // fixed partitions: one record per partition
  int64_t rec_cap = 0;  // piece records in the workspace
  size_t desc_bytes = 0, rec_ml_bytes = 0, rec_o_bytes = 0, ws_bytes = 0;
};

void size_records(Geom& g, int head_dim) {
  g.rec_ml_bytes = align256(static_cast<size_t>(g.rec_cap) * g.rec_rows * sizeof(float));
  g.rec_o_bytes = align256(static_cast<size_t>(g.rec_cap) * g.rec_rows * head_dim * sizeof(float));
  g.ws_bytes = g.desc_bytes + 2 * g.rec_ml_bytes + g.rec_o_bytes;
}

Geom geometry(int64_t num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
              int max_context_len, int partition_size, int dtype) {
  Geom g;
  const int group = num_q_heads / num_kv_heads;
  g.gt = group_tile(group, dtype);
  g.n_gtiles = (group + g.gt - 1) / g.gt;
  g.n_units = num_kv_heads * g.n_gtiles;
  g.w_cap = kMaxWaves;
  g.rec_rows = g.gt < group ? g.gt : group;
  g.desc_bytes = align256(static_cast<size_t>(num_seqs) * g.n_units * 2 * sizeof(int));
  // default split: a head and a tail record per wave; partitions: one per partition, at most
  // ceil(max_ctx / partition_size) per segment
  g.part = partition_size > 0 ? 1 : 0;
  g.rec_cap = g.part ? std::max<int64_t>(1, num_seqs * g.n_units *
                                                ((static_cast<int64_t>(max_context_len) + partition_size - 1) /
                                                 partition_size))
                     : static_cast<int64_t>(2) * g.w_cap;
  size_records(g, head_dim);
  return g;
}

// The same layout for exactly `waves` waves (at most g.w_cap): the smallest scratch one
// launch of that many waves needs (the per-partition records do not depend on the waves).
Geom with_waves(Geom g, int waves, int head_dim) {
  g.w_cap = waves;
  if (!g.part) g.rec_cap = static_cast<int64_t>(2) * waves;
  size_records(g, head_dim);
  return g;
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
  bool kv_fp8 = false;  // pools hold E4M3 codes (q and out are fp16)
  float k_scale = 1.0f, v_scale = 1.0f;
  const pa_vkv* dense = nullptr;  // the virtually contiguous cache instead of pools and tables
  const void* k_new = nullptr;    // append mode: the new tokens' K and V rows
  const void* v_new = nullptr;
};

// need_ws false: every check but the workspace's (the caller brings its own scratch)
int check_decode(const DecodeCall& c, Geom* g, bool need_ws = true) {
  int rc = check_common(c.dtype, c.head_dim, c.block_size);
  if (rc != PA_OK) return rc;
  if (!(c.scale > 0.0f) || !std::isfinite(c.scale))
    return fail(PA_ERR_INVALID_ARG, "scale %g must be positive and finite", static_cast<double>(c.scale));
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
  if (c.partition_size < 0 || c.partition_size % c.block_size != 0 || c.partition_size % 16 != 0)
    return fail(PA_ERR_INVALID_ARG,
                "partition_size %d must be 0 or a positive multiple of 16 and of block_size %d",
                c.partition_size, c.block_size);
  if (c.num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d > 65535", c.num_seqs);
  if (c.num_q_heads > 65535) return fail(PA_ERR_INVALID_ARG, "num_q_heads %d > 65535", c.num_q_heads);
  *g = geometry(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim, c.max_context_len, c.partition_size,
                c.dtype);
  // tile counts, segment indexes and the work split's cost positions (tiles plus pieces)
  // are 32-bit in the kernels (a tile holds at least 8 tokens; every segment counts once
  // besides, or once per partition with fixed partitions, since the split and the reduce
  // count all of them)
  const int64_t mcl = c.max_context_len;
  const int64_t pieces = c.partition_size > 0 ? std::max<int64_t>(1, (mcl + c.partition_size - 1) / c.partition_size) : 1;
  if (static_cast<int64_t>(c.num_seqs) * g->n_units * ((mcl + 7) / 8 + pieces) > (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "batch too large: more than 2^31 - 1 tiles and pieces");
  if (g->rec_cap * g->rec_rows > (static_cast<int64_t>(1) << 31) - 1)  // record rows are 32-bit indexes
    return fail(PA_ERR_INVALID_ARG, "too many partitions: %lld records of %d rows", (long long)g->rec_cap,
                g->rec_rows);
  if (c.num_blocks > (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "num_blocks above 2^31 - 1");
  if (static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim * (c.kv_fp8 ? 1 : c.dtype == PA_F16 ? 2 : 4) >
      (static_cast<int64_t>(1) << 32) - 1)
    return fail(PA_ERR_INVALID_ARG, "one block of one layer exceeds 4 GiB");
  if (c.num_seqs == 0) return PA_OK;
  if (!c.out || !c.q || !c.k_cache || !c.v_cache || !c.block_tables || !c.context_lens)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(c.out, 16) || !aligned(c.q, 16) || !aligned(c.k_cache, 16) || !aligned(c.v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "out, q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(c.block_tables, 4) || !aligned(c.context_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables and context_lens must be 4-byte aligned");
  if (need_ws) {
    if (!c.workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", g->ws_bytes);
    if (c.workspace_bytes < g->ws_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", c.workspace_bytes, g->ws_bytes);
    if (!aligned(c.workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (c.k_new || c.v_new) {
    if (!c.k_new || !c.v_new) return fail(PA_ERR_INVALID_ARG, "k_new or v_new is NULL");
    if (!aligned(c.k_new, 16) || !aligned(c.v_new, 16))
      return fail(PA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  }
  return PA_OK;
}

struct WsParts {
  int2* desc;
  float* rec_m;
  float* rec_l;
  float* rec_o;
};

WsParts split_workspace(void* ws, const Geom& g) {
  char* b = static_cast<char*>(ws);
  WsParts p;
  p.desc = reinterpret_cast<int2*>(b);
  b += g.desc_bytes;
  p.rec_m = reinterpret_cast<float*>(b);
  p.rec_l = reinterpret_cast<float*>(b + g.rec_ml_bytes);
  p.rec_o = reinterpret_cast<float*>(b + 2 * g.rec_ml_bytes);
  return p;
}

// Resident one-wave work-groups of a kernel on the current device, and the device's
// compute units (cached per device and kernel: fixed for a given build and device).
struct Residency {
  int waves = 0, cus = 0;
};

// Resident waves of a one-wave kernel on the current device, memoised per (device, kernel).
// A full table only stops the memoising: the answer is the same either way, since the work
// split, and with it the rounding of every split context, depends on it.  {0, 0} if the
// runtime cannot say.
Residency residency(const void* kernel) {
  constexpr int kSlots = 32;
  static std::mutex mu;
  static const void* keys[64][kSlots] = {};
  static Residency vals[64][kSlots];
  int dev = 0;
  Residency r;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return r;
  }
  std::lock_guard<std::mutex> lock(mu);
  int slot = -1;
  for (int i = 0; i < kSlots; ++i) {
    if (keys[dev][i] == kernel) return vals[dev][i];
    if (keys[dev][i] == nullptr) {
      slot = i;
      break;
    }
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWave, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu <= 0 ||
      cus <= 0) {
    (void)hipGetLastError();
    return r;
  }
  r.waves = per_cu * cus;
  r.cus = cus;
  if (slot >= 0) {
    keys[dev][slot] = kernel;
    vals[dev][slot] = r;
  }
  return r;
}

// The odd-numbered waves' share weight: kOddDieWeight on a whole device, else equal weights.
int die_weight(const void* kernel) { return residency(kernel).cus == kWholeDeviceCUs ? kOddDieWeight : 64; }

// Waves of one launch: `base`, never more than the workspace allows.
int waves_for(const DecodeCall&, const Geom& g, int64_t base) {
  int64_t w = base > 0 ? base : kMaxWaves;
  if (w > g.w_cap) w = g.w_cap;
  return static_cast<int>(w < 1 ? 1 : w);
}

// fp32: every resident wave (at most kMaxWaves).  fp16: kMfWavesPerCU per compute unit:
// a few deep streams per unit keep HBM busy with less contention than a full unit.
// E4M3 pools: kF8WavesPerCU shallower streams.
// Both return 0 when the residency query fails (the launch then reports an error rather than
// pick another split).
template <typename T, int D, int GT>
int waves_valu(const DecodeCall& c, const Geom& g) {
  const Residency r = residency(reinterpret_cast<const void*>(pa_stream_kernel<T, D, GT>));
  if (r.waves <= 0) return 0;
  return waves_for(c, g, r.waves > kMaxWaves ? kMaxWaves : r.waves);
}

template <int D, int NST, bool F8, bool DENSE, bool APPEND>
int waves_mfma(const DecodeCall& c, const Geom& g, int waves_per_cu) {
  const Residency r = residency(reinterpret_cast<const void*>(pa_stream_mfma_kernel<D, NST, F8, DENSE, APPEND>));
  if (r.waves <= 0) return 0;
  int64_t base = static_cast<int64_t>(r.cus) * waves_per_cu;
  if (base > r.waves) base = r.waves;
  return waves_for(c, g, base);
}

StreamArgs stream_args(const DecodeCall& c, const Geom& g) {
  const WsParts ws = split_workspace(c.workspace, g);
  StreamArgs a;
  a.out = c.out;
  a.seg_desc = ws.desc;
  a.rec_m = ws.rec_m;
  a.rec_l = ws.rec_l;
  a.rec_o = ws.rec_o;
  a.q = c.q;
  a.k_cache = c.k_cache;
  a.v_cache = c.v_cache;
  a.block_tables = c.block_tables;
  a.context_lens = c.context_lens;
  // E4M3 pools: the K scale multiplies every score, so it joins the softmax scale
  a.scale_log2 = static_cast<float>(static_cast<double>(c.scale) * (c.kv_fp8 ? c.k_scale : 1.0) *
                                    1.4426950408889634);
  a.out_scale = c.kv_fp8 ? c.v_scale : 1.0f;
  a.block_size = c.block_size;
  a.log2_block = log2_of(c.block_size);
  a.num_kv_heads = c.num_kv_heads;
  a.num_q_heads = c.num_q_heads;
  a.group = c.num_q_heads / c.num_kv_heads;
  a.n_gtiles = g.n_gtiles;
  a.n_units = g.n_units;
  a.num_seqs = c.num_seqs;
  a.max_blocks_per_seq = c.max_blocks_per_seq;
  a.max_context_len = c.max_context_len;
  a.num_blocks = c.num_blocks;
  a.num_waves = 1;
  a.rec_rows = g.rec_rows;
  a.part_tiles = 0;  // set by the launch, from its kernel's tile
  a.odd_weight = 64;  // set by the launch, from the device
  a.dense_k = a.dense_v = a.guard_k = a.guard_v = nullptr;
  a.seq_bytes = a.token_bytes = 0;
  if (c.dense) {
    a.dense_k = c.dense->k_base();
    a.dense_v = c.dense->v_base();
    a.guard_k = c.dense->k_reserve;
    a.guard_v = c.dense->v_reserve;
    a.seq_bytes = c.dense->seq_bytes;
    a.token_bytes = c.dense->token_bytes;
  }
  a.k_new = static_cast<const char*>(c.k_new);
  a.v_new = static_cast<const char*>(c.v_new);
  a.k_sc = f8_scale(c.k_scale);
  a.v_sc = f8_scale(c.v_scale);
  return a;
}

template <typename T, int D, int GT>
int launch_stream(const DecodeCall& c, const Geom& g) {
  StreamArgs a = stream_args(c, g);
  a.part_tiles = c.partition_size / Cfg<T, D, GT>::kTK;  // a multiple of 16 tokens: whole tiles
  a.num_waves = waves_valu<T, D, GT>(c, g);
  a.odd_weight = die_weight(reinterpret_cast<const void*>(pa_stream_kernel<T, D, GT>));
  if (a.num_waves <= 0) return fail(PA_ERR_HIP, "occupancy query for pa_stream_kernel failed");
  hipLaunchKernelGGL((pa_stream_kernel<T, D, GT>), dim3(a.num_waves), dim3(kWave), 0, c.stream, a);
  return check_hip("pa_stream_kernel launch");
}

// NST stages, waves_per_cu waves per compute unit
template <int D, int NST, bool F8, bool DENSE = false, bool APPEND = false>
int launch_stream_mfma(const DecodeCall& c, const Geom& g, int waves_per_cu) {
  StreamArgs a = stream_args(c, g);
  a.part_tiles = c.partition_size / MCfg<D, F8>::kTK;  // a multiple of 16 tokens: whole tiles
  a.num_waves = waves_mfma<D, NST, F8, DENSE, APPEND>(c, g, waves_per_cu);
  a.odd_weight = die_weight(reinterpret_cast<const void*>(pa_stream_mfma_kernel<D, NST, F8, DENSE, APPEND>));
  if (a.num_waves <= 0) return fail(PA_ERR_HIP, "occupancy query for pa_stream_mfma_kernel failed");
  hipLaunchKernelGGL((pa_stream_mfma_kernel<D, NST, F8, DENSE, APPEND>), dim3(a.num_waves), dim3(kWave), 0, c.stream,
                     a);
  return check_hip("pa_stream_mfma_kernel launch");
}

template <typename T, int D, int GT>
int launch_reduce(const DecodeCall& c, const Geom& g) {
  const WsParts ws = split_workspace(c.workspace, g);
  AppendArgs ap{};  // k_new == nullptr: the reduce writes no cache row
  if (c.k_new) {
    ap.k_new = static_cast<const char*>(c.k_new);
    ap.v_new = static_cast<const char*>(c.v_new);
    ap.k_cache = static_cast<char*>(const_cast<void*>(c.k_cache));
    ap.v_cache = static_cast<char*>(const_cast<void*>(c.v_cache));
    ap.block_tables = c.block_tables;
    ap.max_blocks_per_seq = c.max_blocks_per_seq;
    ap.block_size = c.block_size;
    ap.num_kv_heads = c.num_kv_heads;
    ap.num_blocks = c.num_blocks;
    ap.codes = c.kv_fp8 ? 1 : 0;
    ap.k_sc = f8_scale(c.k_scale);
    ap.v_sc = f8_scale(c.v_scale);
  }
  hipLaunchKernelGGL((pa_reduce_kernel<T, D, GT>), dim3(c.num_q_heads, c.num_seqs), dim3(kWave), 0,
                     c.stream, static_cast<T*>(c.out), ws.desc, ws.rec_m, ws.rec_l, ws.rec_o,
                     c.context_lens, c.num_q_heads, c.num_q_heads / c.num_kv_heads, g.n_gtiles,
                     c.max_context_len, g.w_cap, g.rec_rows, g.part, g.rec_cap, ap);
  return check_hip("pa_reduce_kernel launch");
}

template <int Which, int D>
int dispatch_f32(const DecodeCall& c, const Geom& g) {
  switch (g.gt) {
    case 1: return Which == 0 ? launch_stream<float, D, 1>(c, g) : launch_reduce<float, D, 1>(c, g);
    case 2: return Which == 0 ? launch_stream<float, D, 2>(c, g) : launch_reduce<float, D, 2>(c, g);
    case 4: return Which == 0 ? launch_stream<float, D, 4>(c, g) : launch_reduce<float, D, 4>(c, g);
    default: return Which == 0 ? launch_stream<float, D, 8>(c, g) : launch_reduce<float, D, 8>(c, g);
  }
}

template <int Which, int D>
int dispatch_f16(const DecodeCall& c, const Geom& g) {
  if (Which == 1) return launch_reduce<f16, D, kMfRows>(c, g);
  if (c.dense) return launch_stream_mfma<D, kMfStages, false, true>(c, g, kMfWavesPerCU);
  if (c.k_new)
    return c.kv_fp8 ? launch_stream_mfma<D, kF8Stages, true, false, true>(c, g, kF8WavesPerCU)
                    : launch_stream_mfma<D, kMfStages, false, false, true>(c, g, kMfWavesPerCU);
  return c.kv_fp8 ? launch_stream_mfma<D, kF8Stages, true>(c, g, kF8WavesPerCU)
                  : launch_stream_mfma<D, kMfStages, false>(c, g, kMfWavesPerCU);
}

// Which = 0: the stream kernel; 1: the reduce kernel
template <int Which>
int dispatch(const DecodeCall& c, const Geom& g) {
  if (c.num_seqs == 0) return PA_OK;
  if (c.dtype == PA_F16)
    return c.head_dim == 64 ? dispatch_f16<Which, 64>(c, g) : dispatch_f16<Which, 128>(c, g);
  return c.head_dim == 64 ? dispatch_f32<Which, 64>(c, g) : dispatch_f32<Which, 128>(c, g);
}

// A launch's work-items are counted in 32 bits: one thread per 16-byte chunk (fp16/fp32
// pools) or per 16 codes (E4M3 pools), in whole work-groups of 256.
constexpr int64_t kMaxWriteThreads = (static_cast<int64_t>(1) << 31) - 256;

template <typename T, int D>
int launch_cache_write(const void* k, const void* v, const int64_t* slots, void* kc, void* vc,
                       int num_tokens, int num_kv_heads, int block_size, int64_t num_blocks,
                       hipStream_t stream) {
  constexpr int kChunksPerRow = D * static_cast<int>(sizeof(T)) / 16;
  const int64_t chunks = static_cast<int64_t>(num_tokens) * num_kv_heads * kChunksPerRow;
  if (chunks > kMaxWriteThreads)
    return fail(PA_ERR_INVALID_ARG, "%lld 16-byte chunks in one write; at most %lld (split the tokens)",
                (long long)chunks, (long long)kMaxWriteThreads);
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL((pa_cache_write_kernel<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const T*>(k), static_cast<const T*>(v), slots,
                     static_cast<T*>(kc), static_cast<T*>(vc), chunks, num_kv_heads, block_size,
                     num_blocks * block_size);
  return check_hip("pa_cache_write_kernel launch");
}

template <int D>
int launch_cache_write_fp8(const void* k, const void* v, const int64_t* slots, void* kc, void* vc,
                           F8Scale ks, F8Scale vs, int num_tokens, int num_kv_heads, int block_size,
                           int64_t num_blocks, hipStream_t stream) {
  const int64_t chunks = static_cast<int64_t>(num_tokens) * num_kv_heads * (D / 16);
  if (chunks > kMaxWriteThreads)
    return fail(PA_ERR_INVALID_ARG, "%lld threads in one write; at most %lld (split the tokens)",
                (long long)chunks, (long long)kMaxWriteThreads);
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL((pa_cache_write_fp8_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const f16*>(k), static_cast<const f16*>(v), slots,
                     static_cast<uint8_t*>(kc), static_cast<uint8_t*>(vc), ks, vs, chunks,
                     num_kv_heads, block_size, num_blocks * block_size);
  return check_hip("pa_cache_write_fp8_kernel launch");
}

bool valid_scale(float x) { return x > 0.0f && std::isfinite(x); }

// Grid order.  When chunks make up at least half their context (whole prompts), the causal
// row blocks differ most in length: row blocks outermost starts the longest ones of every
// sequence and head first, which balances the compute units (Llama-2-70B prompts: 12 %
// faster).  After a long cached prefix the blocks differ less, and keeping the row blocks of
// one (sequence, kv head) together, which share its K/V in the caches, is faster (7 %).
template <int D, int NR>
int launch_prefill_rows(PrefillArgs a, int64_t rows, int num_seqs, hipStream_t stream) {
  constexpr int kRows = kPfWaves * NR * 16;
  a.n_row_blocks = static_cast<int>((rows + kRows - 1) / kRows);
  a.rb_outer = 2 * static_cast<int64_t>(a.max_query_len) >= a.max_context_len && a.n_row_blocks <= 65535 ? 1 : 0;
  const dim3 grid = a.rb_outer ? dim3(a.num_kv_heads, num_seqs, a.n_row_blocks)
                               : dim3(a.n_row_blocks, a.num_kv_heads, num_seqs);
  hipLaunchKernelGGL((pa_prefill_kernel<D, NR, kPfStages>), grid, dim3(kPfWaves * kWave), 0, stream, a);
  return check_hip("pa_prefill_kernel launch");
}

// 32 rows per wave (two 16-row blocks) with the kernel held to 256 registers, so that two
// waves share each SIMD and one's softmax runs beside the other's products, and a 2-stage
// ring: measured fastest on MI355X both for chunks after a long cached prefix and for whole
// prompts (64 rows per wave needs more registers and runs one wave per SIMD).
template <int D>
int launch_prefill(const PrefillArgs& a, int64_t rows, int num_seqs, hipStream_t stream) {
  return launch_prefill_rows<D, kPfBlocks>(a, rows, num_seqs, stream);
}

// Waves of pa_decode's stream launch for these sizes on the current device (0 if the
// occupancy query fails): the split the launch itself will pick.
template <int D>
int decode_waves(const DecodeCall& c, const Geom& g) {
  if (c.dtype == PA_F16) return waves_mfma<D, kMfStages, false, false, false>(c, g, kMfWavesPerCU);
  switch (g.gt) {
    case 1: return waves_valu<float, D, 1>(c, g);
    case 2: return waves_valu<float, D, 2>(c, g);
    case 4: return waves_valu<float, D, 4>(c, g);
    default: return waves_valu<float, D, 8>(c, g);
  }
}

// Scratch of pa_decode_noalloc: segment descriptors and piece records, laid out as a
// workspace.  One copy per GPU, held until the process ends; no call needs it cleared (every
// descriptor and record a call reads, the same call wrote first).
constexpr size_t kScratchBytes = static_cast<size_t>(PA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per device with that
// device current (each GPU holds its own copy at its own address).  In host code the name
// `scratch` is only a stand-in: kernels and copies must be given this address.
int scratch_address(void** out) {
  constexpr int kDevs = 64;
  static std::mutex mu;
  static void* addr[kDevs] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) {
    (void)hipGetLastError();
    return fail(PA_ERR_HIP, "no current device (or device index %d above %d)", dev, kDevs - 1);
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return PA_OK;
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

// ---- pa_decode_shared: geometry, checks, launches

// Workspace of pa_decode_shared: a descriptor per (virtual sequence, kv head), and records
// of kShRows rows: two per wave (of at most kMaxWaves) for split segments, one per segment
// for segments held whole by one wave.
Geom shared_geometry(int64_t num_seqs, int64_t num_groups, int num_kv_heads, int head_dim) {
  Geom g;
  g.gt = kMfRows;
  g.n_gtiles = 1;
  g.n_units = num_kv_heads;
  g.rec_rows = kShRows;
  g.w_cap = kMaxWaves;
  const int64_t segs = (num_groups + num_seqs) * num_kv_heads;
  const int64_t recs = 2 * static_cast<int64_t>(g.w_cap) + segs;
  g.desc_bytes = align256(static_cast<size_t>(segs) * 2 * sizeof(int));
  g.rec_ml_bytes = align256(static_cast<size_t>(recs) * g.rec_rows * sizeof(float));
  g.rec_o_bytes = align256(static_cast<size_t>(recs) * g.rec_rows * head_dim * sizeof(float));
  g.ws_bytes = g.desc_bytes + 2 * g.rec_ml_bytes + g.rec_o_bytes;
  return g;
}

// launches: bit 0 the stream kernel, bit 1 the reduce
template <int D>
int launch_shared(const DecodeCall& c, const Geom& g, const SharedArgs& sh, int launches) {
  const Residency r = residency(reinterpret_cast<const void*>(pa_shared_mfma_kernel<D>));
  if (r.waves <= 0) return fail(PA_ERR_HIP, "occupancy query for pa_shared_mfma_kernel failed");
  int64_t waves = static_cast<int64_t>(r.cus) * kShWavesPerCU;
  if (waves > r.waves) waves = r.waves;
  if (waves > g.w_cap) waves = g.w_cap;
  StreamArgs a = stream_args(c, g);
  a.num_waves = static_cast<int>(waves);
  if (launches & 1) {
    hipLaunchKernelGGL((pa_shared_mfma_kernel<D>), dim3(a.num_waves), dim3(kWave), 0, c.stream, a, sh);
    const int rc = check_hip("pa_shared_mfma_kernel launch");
    if (rc != PA_OK) return rc;
  }
  if (launches & 2) {
    const WsParts ws = split_workspace(c.workspace, g);
    hipLaunchKernelGGL((pa_shared_reduce_kernel<D>), dim3(c.num_q_heads, c.num_seqs), dim3(kWave), 0, c.stream,
                       static_cast<f16*>(c.out), ws.desc, ws.rec_m, ws.rec_l, ws.rec_o, c.context_lens, sh,
                       c.num_seqs, c.num_q_heads, c.num_q_heads / c.num_kv_heads, g.n_units, c.max_context_len,
                       c.block_size, a.num_waves, g.rec_rows);
    return check_hip("pa_shared_reduce_kernel launch");
  }
  return PA_OK;
}

int decode_shared(int launches, void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_group,
                  const int32_t* group_first, const int32_t* group_size, const int32_t* group_prefix,
                  int32_t num_groups, float scale, int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                  int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                  int64_t num_blocks, void* workspace, size_t workspace_bytes, void* stream) {
  g_error.clear();
  DecodeCall c = make_call(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, num_kv_heads,
                           num_seqs, num_q_heads, head_dim, max_blocks_per_seq, max_context_len, num_blocks, 0,
                           PA_F16, workspace, workspace_bytes, stream);
  Geom g0;
  int rc = check_decode(c, &g0, false);
  if (rc != PA_OK) return rc;
  if (num_q_heads / num_kv_heads > kMfRows)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_shared: %d query heads per kv head, at most %d",
                num_q_heads / num_kv_heads, kMfRows);
  if (num_groups < 0 || num_groups > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_groups %d outside [0, 65535]", num_groups);
  if ((static_cast<int64_t>(num_seqs) + num_groups) * num_kv_heads *
          std::max<int64_t>(1, (static_cast<int64_t>(max_context_len) + 7) / 8) >
      (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "batch too large: more than 2^31 - 1 tiles or segments");
  // the work split's cost positions are 32-bit
  if ((static_cast<int64_t>(num_seqs) + num_groups) * num_kv_heads *
          (kShSegCost + kShTileCost2 * ((static_cast<int64_t>(max_context_len) + 15) / 16)) >
      (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "batch too large for the shared-prefix work split");
  if (num_seqs == 0) return PA_OK;
  if (!seq_group || (num_groups > 0 && (!group_first || !group_size || !group_prefix)))
    return fail(PA_ERR_INVALID_ARG, "a group array is NULL");
  if (!aligned(seq_group, 4) || !aligned(group_first, 4) || !aligned(group_size, 4) || !aligned(group_prefix, 4))
    return fail(PA_ERR_INVALID_ARG, "the group arrays must be 4-byte aligned");
  const Geom g = shared_geometry(num_seqs, num_groups, num_kv_heads, head_dim);
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", g.ws_bytes);
  if (workspace_bytes < g.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, g.ws_bytes);
  if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const SharedArgs sh{seq_group, group_first, group_size, group_prefix, num_groups};
  return head_dim == 64 ? launch_shared<64>(c, g, sh, launches) : launch_shared<128>(c, g, sh, launches);
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

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || partition_size < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  // the larger of the two layouts, so one workspace serves either element type
  const size_t a = geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size,
                            PA_F32).ws_bytes;
  const size_t b = geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size,
                            PA_F16).ws_bytes;
  return a > b ? a : b;
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
  Geom g;
  const int rc = check_decode(c, &g);
  if (rc != PA_OK) return rc;
  return dispatch<0>(c, g);
}

int pa_decode_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t max_context_len, int32_t partition_size, int32_t dtype,
                     const void* workspace, size_t workspace_bytes, void* stream) {
  g_error.clear();
  if (dtype != PA_F32 && dtype != PA_F16) return fail(PA_ERR_UNSUPPORTED, "dtype %d is not PA_F32 or PA_F16", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", head_dim);
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 || partition_size < 0)
    return fail(PA_ERR_INVALID_ARG, "negative or zero size");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, num_kv_heads);
  if (num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d > 65535", num_seqs);
  if (num_q_heads > 65535) return fail(PA_ERR_INVALID_ARG, "num_q_heads %d > 65535", num_q_heads);
  if (partition_size % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "partition_size %d must be 0 or a positive multiple of 16", partition_size);
  if (num_seqs == 0) return PA_OK;
  const Geom g = geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size, dtype);
  if (static_cast<int64_t>(num_seqs) * g.n_units > (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "batch too large: more than 2^31 - 1 segments");
  if (g.rec_cap * g.rec_rows > (static_cast<int64_t>(1) << 31) - 1)  // record rows are 32-bit indexes
    return fail(PA_ERR_INVALID_ARG, "too many partitions: %lld records of %d rows", (long long)g.rec_cap,
                g.rec_rows);
  if (!out || !context_lens) return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(out, 16) || !aligned(context_lens, 4)) return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", g.ws_bytes);
  if (workspace_bytes < g.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, g.ws_bytes);
  if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  DecodeCall c{};
  c.out = out;
  c.context_lens = context_lens;
  c.num_seqs = num_seqs;
  c.num_q_heads = num_q_heads;
  c.num_kv_heads = num_kv_heads;
  c.head_dim = head_dim;
  c.max_context_len = max_context_len;
  c.partition_size = partition_size;
  c.dtype = dtype;
  c.workspace = const_cast<void*>(workspace);
  c.workspace_bytes = workspace_bytes;
  c.stream = static_cast<hipStream_t>(stream);
  return dispatch<1>(c, g);
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
  Geom g;
  int rc = check_decode(c, &g);
  if (rc != PA_OK) return rc;
  rc = dispatch<0>(c, g);
  if (rc != PA_OK) return rc;
  return dispatch<1>(c, g);
}

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                      int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                      int64_t num_blocks, int32_t partition_size, int32_t dtype, void* stream) {
  g_error.clear();
  DecodeCall c = make_call(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                           num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                           max_context_len, num_blocks, partition_size, dtype, nullptr, 0, stream);
  Geom g;
  int rc = check_decode(c, &g, false);
  if (rc != PA_OK || c.num_seqs == 0) return rc;
  const int waves = head_dim == 64 ? decode_waves<64>(c, g) : decode_waves<128>(c, g);
  if (waves <= 0) return fail(PA_ERR_HIP, "occupancy query for the decode kernel failed");
  const Geom gs = with_waves(g, waves, head_dim);
  if (gs.ws_bytes > kScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "these sizes need %zu bytes of scratch, above the %zu this call holds; use pa_decode "
                "with a workspace",
                gs.ws_bytes, kScratchBytes);
  rc = scratch_address(&c.workspace);
  if (rc != PA_OK) return rc;
  c.workspace_bytes = kScratchBytes;
  rc = dispatch<0>(c, gs);
  if (rc != PA_OK) return rc;
  return dispatch<1>(c, gs);
}

static int decode_append(int launches, void* out, const void* q, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, int32_t block_size, int32_t num_kv_heads,
                         int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int64_t num_blocks, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_error.clear();
  DecodeCall c = make_call(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                           num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                           max_context_len, num_blocks, partition_size, PA_F16, workspace, workspace_bytes,
                           stream);
  c.k_new = k_new;
  c.v_new = v_new;
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, "k_new or v_new is NULL");
  Geom g;
  int rc = check_decode(c, &g);
  if (rc != PA_OK) return rc;
  rc = dispatch<0>(c, g);
  if (rc != PA_OK || launches == 1) return rc;
  return dispatch<1>(c, g);
}

int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                     void* v_cache, const int32_t* block_tables, const int32_t* context_lens, float scale,
                     int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                     int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                     int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_append(2, out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq, max_context_len,
                       num_blocks, partition_size, workspace, workspace_bytes, stream);
}

int pa_decode_append_partitions(void* out, const void* q, const void* k_new, const void* v_new,
                                const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, float scale, int32_t block_size,
                                int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                                int32_t partition_size, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_append(1, out, q, k_new, v_new, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                       block_tables, context_lens, scale, block_size, num_kv_heads, num_seqs, num_q_heads,
                       head_dim, max_blocks_per_seq, max_context_len, num_blocks, partition_size, workspace,
                       workspace_bytes, stream);
}

int pa_cache_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                       void* v_cache, float k_scale, float v_scale, int32_t num_tokens,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                       void* stream) {
  g_error.clear();
  int rc = check_common(PA_F16, head_dim, block_size);
  if (rc != PA_OK) return rc;
  if (!valid_scale(k_scale) || !valid_scale(v_scale))
    return fail(PA_ERR_INVALID_ARG, "k_scale %g and v_scale %g must be positive and finite",
                static_cast<double>(k_scale), static_cast<double>(v_scale));
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d must be > 0", num_kv_heads);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld must be > 0", (long long)num_blocks);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "k, v, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(PA_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  const F8Scale k_sc = f8_scale(k_scale);
  const F8Scale v_sc = f8_scale(v_scale);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64
             ? launch_cache_write_fp8<64>(k, v, slot_mapping, k_cache, v_cache, k_sc, v_sc, num_tokens,
                                          num_kv_heads, block_size, num_blocks, st)
             : launch_cache_write_fp8<128>(k, v, slot_mapping, k_cache, v_cache, k_sc, v_sc, num_tokens,
                                           num_kv_heads, block_size, num_blocks, st);
}

// k_new == nullptr: pa_decode_fp8; otherwise the append form (new fp16 rows in k_new / v_new)
static int decode_fp8(int launches, const void* k_new, const void* v_new, void* out, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, float k_scale, float v_scale,
                      int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                      int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  g_error.clear();
  DecodeCall c = make_call(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                           num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                           max_context_len, num_blocks, partition_size, PA_F16, workspace, workspace_bytes,
                           stream);
  c.kv_fp8 = true;
  c.k_scale = k_scale;
  c.v_scale = v_scale;
  c.k_new = k_new;
  c.v_new = v_new;
  if (!valid_scale(k_scale) || !valid_scale(v_scale))
    return fail(PA_ERR_INVALID_ARG, "k_scale %g and v_scale %g must be positive and finite",
                static_cast<double>(k_scale), static_cast<double>(v_scale));
  if (!valid_scale(static_cast<float>(static_cast<double>(scale) * k_scale)))
    return fail(PA_ERR_INVALID_ARG, "scale * k_scale is not a positive finite fp32 value");
  Geom g;
  int rc = check_decode(c, &g);
  if (rc != PA_OK) return rc;
  rc = dispatch<0>(c, g);
  if (rc != PA_OK || launches == 1) return rc;
  return dispatch<1>(c, g);
}

int pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, float scale, float k_scale,
                  float v_scale, int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                  int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                  int32_t max_context_len, int64_t num_blocks, int32_t partition_size, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return decode_fp8(2, nullptr, nullptr, out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                    v_scale,
                    block_size, num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                    max_context_len, num_blocks, partition_size, workspace, workspace_bytes, stream);
}

int pa_decode_fp8_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, float scale,
                             float k_scale, float v_scale, int32_t block_size, int32_t num_kv_heads,
                             int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                             int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                             int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_fp8(1, nullptr, nullptr, out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                    v_scale,
                    block_size, num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                    max_context_len, num_blocks, partition_size, workspace, workspace_bytes, stream);
}

int pa_decode_fp8_append(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, const int32_t* block_tables, const int32_t* context_lens, float scale,
                         float k_scale, float v_scale, int32_t block_size, int32_t num_kv_heads,
                         int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int64_t num_blocks, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) {
    g_error.clear();
    return fail(PA_ERR_INVALID_ARG, "k_new or v_new is NULL");
  }
  return decode_fp8(2, k_new, v_new, out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                    v_scale, block_size, num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                    max_context_len, num_blocks, partition_size, workspace, workspace_bytes, stream);
}

int pa_decode_fp8_append_partitions(void* out, const void* q, const void* k_new, const void* v_new,
                                    const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, float scale, float k_scale, float v_scale,
                                    int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t max_context_len, int64_t num_blocks, int32_t partition_size,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) {
    g_error.clear();
    return fail(PA_ERR_INVALID_ARG, "k_new or v_new is NULL");
  }
  return decode_fp8(1, k_new, v_new, out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                    v_scale, block_size, num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                    max_context_len, num_blocks, partition_size, workspace, workspace_bytes, stream);
}

int pa_decode_dense(void* out, const void* q, const pa_vkv* kv, float scale, int32_t num_q_heads,
                    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  g_error.clear();
  if (!kv) return fail(PA_ERR_INVALID_ARG, "NULL cache");
  if (!valid_scale(scale))
    return fail(PA_ERR_INVALID_ARG, "scale %g must be positive and finite", static_cast<double>(scale));
  if (num_q_heads <= 0 || num_q_heads % kv->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d", num_q_heads,
                kv->num_kv_heads);
  if (partition_size < 0 || partition_size % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "partition_size %d must be 0 or a positive multiple of 16", partition_size);
  const int32_t num_seqs = kv->num_seqs;
  if (num_seqs == 0) return PA_OK;
  const Geom g = geometry(num_seqs, num_q_heads, kv->num_kv_heads, kv->head_dim, kv->max_ctx, partition_size, PA_F16);
  if (static_cast<int64_t>(num_seqs) * g.n_units * ((static_cast<int64_t>(kv->max_ctx) + 15) / 16) >
      (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "batch too large: more than 2^31 - 1 tiles");
  if (!out || !q) return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(out, 16) || !aligned(q, 16)) return fail(PA_ERR_INVALID_ARG, "out and q must be 16-byte aligned");
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", g.ws_bytes);
  if (workspace_bytes < g.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, g.ws_bytes);
  if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  DecodeCall c = make_call(out, q, nullptr, nullptr, nullptr, kv->d_ctx, scale, 16, kv->num_kv_heads, num_seqs,
                           num_q_heads, kv->head_dim, 0, kv->max_ctx, 0, partition_size, PA_F16, workspace,
                           workspace_bytes, stream);
  c.dense = kv;
  int rc = dispatch<0>(c, g);
  if (rc != PA_OK) return rc;
  return dispatch<1>(c, g);
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
               float scale, int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
               int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
               int32_t max_query_len, int32_t max_context_len, int64_t num_blocks, int32_t dtype,
               void* stream) {
  g_error.clear();
  int rc = check_common(dtype, head_dim, block_size);
  if (rc != PA_OK) return rc;
  if (dtype != PA_F16) return fail(PA_ERR_UNSUPPORTED, "pa_prefill is built for PA_F16 only");
  if (!valid_scale(scale))
    return fail(PA_ERR_INVALID_ARG, "scale %g must be positive and finite", static_cast<double>(scale));
  if (num_seqs < 0 || max_query_len < 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "num_seqs, max_query_len and max_context_len must be >= 0");
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d must be > 0", max_blocks_per_seq);
  if (num_blocks <= 0 || num_blocks > (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "num_blocks %lld outside [1, 2^31 - 1]", (long long)num_blocks);
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len %d exceeds max_blocks_per_seq * block_size", max_context_len);
  if (num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d > 65535", num_seqs);
  if (num_q_heads > 65535) return fail(PA_ERR_INVALID_ARG, "num_q_heads %d > 65535", num_q_heads);
  if (static_cast<int64_t>(num_kv_heads) * block_size * head_dim * 2 > (static_cast<int64_t>(1) << 32) - 1)
    return fail(PA_ERR_INVALID_ARG, "one block of one layer exceeds 4 GiB");
  const int group = num_q_heads / num_kv_heads;
  const int64_t rows = static_cast<int64_t>(max_query_len) * group;
  if (rows > (static_cast<int64_t>(1) << 30))
    return fail(PA_ERR_INVALID_ARG, "max_query_len * group above 2^30 rows per sequence");
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "out, q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables, context_lens and query_start must be 4-byte aligned");
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.block_size = block_size;
  a.log2_block = log2_of(block_size);
  a.num_kv_heads = num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.group = group;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.max_context_len = max_context_len;
  a.num_blocks = num_blocks;
  a.n_row_blocks = 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64 ? launch_prefill<64>(a, rows, num_seqs, st) : launch_prefill<128>(a, rows, num_seqs, st);
}

size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_groups, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim) {
  if (num_seqs <= 0 || num_groups < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  return shared_geometry(num_seqs, num_groups, num_kv_heads, head_dim).ws_bytes;
}

int pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* seq_group, const int32_t* group_first,
                     const int32_t* group_size, const int32_t* group_prefix, int32_t num_groups, float scale,
                     int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                     int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_shared(3, out, q, k_cache, v_cache, block_tables, context_lens, seq_group, group_first, group_size,
                       group_prefix, num_groups, scale, block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                       max_blocks_per_seq, max_context_len, num_blocks, workspace, workspace_bytes, stream);
}

int pa_decode_shared_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_group,
                                const int32_t* group_first, const int32_t* group_size, const int32_t* group_prefix,
                                int32_t num_groups, float scale, int32_t block_size, int32_t num_kv_heads,
                                int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                int32_t max_context_len, int64_t num_blocks, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_shared(1, out, q, k_cache, v_cache, block_tables, context_lens, seq_group, group_first, group_size,
                       group_prefix, num_groups, scale, block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                       max_blocks_per_seq, max_context_len, num_blocks, workspace, workspace_bytes, stream);
}

}  // extern "C"

