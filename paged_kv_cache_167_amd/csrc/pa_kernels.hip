// Paged KV-cache decode attention for MI355X (gfx950, CDNA4, wave64).
//
// Three kernels:
//   pa_cache_write_kernel  -- scatter each new token's K/V row into its slot.
//   pa_stream_kernel       -- attention over the paged K/V, the whole batch streamed
//                             by persistent waves that each own an equal share of it.
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
//    ordered by (sequence, kv head, position) and every persistent wave takes an
//    equal, contiguous run of tiles.  A context split between waves leaves one
//    partial result per piece; the reduce kernel merges the pieces by log-sum-exp.
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

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "pa.h"

namespace {

using f16 = _Float16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxWaves = 4096;  // persistent waves in the default split (MI355X holds 2048+)

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

__device__ __forceinline__ int wave_sum_int(int x) {
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ int wave_incl_scan_int(int x, int lane) {
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
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
// decode, pass 1: persistent waves streaming equal shares of the batch
// ---------------------------------------------------------------------------

// A segment is one (sequence, unit) pair, unit = (kv head, tile of GT query heads);
// it has ceil(ctx / TK) tiles.  Segments are ordered by sequence, then unit.
struct StreamArgs {
  void* out;
  int2* seg_desc;  // [S * n_units] {first wave, last wave} holding pieces of the segment
  float* rec_m;    // [2 * W * GT] per piece record: running max (log2 units) per row
  float* rec_l;    // [2 * W * GT] exp-sum per row
  float* rec_o;    // [2 * W * GT * D] normalised output per row
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
};

// Position of a wave in the flattened tile list (all wave-uniform, in SGPRs).
struct Cursor {
  int s;       // sequence
  int unit;    // kv head * n_gtiles + query-head tile
  int t;       // tile within the segment
  int nt;      // tiles in the segment
  int ctx;     // context length of the sequence
  int gstart;  // global index of the segment's first tile
};

template <typename T, int D, int GT>
__global__ __launch_bounds__(kWave) void pa_stream_kernel(const StreamArgs a) {
  using K = Cfg<T, D, GT>;
  constexpr int RK = K::kRK, NL = K::kNL, DL = K::kDL, C = K::kC, E = K::kE, TK = K::kTK;
  constexpr int GR = K::kGroups;
  __shared__ __align__(16) u32x4 s_stage0[8][kWave];
  __shared__ __align__(16) u32x4 s_stage1[8][kWave];

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int sub = lane % C;  // which chunks of a row this lane holds
  const int grp = lane / C;  // which token of a row slot this lane holds
  const int S = a.num_seqs;
  const int32_t* ctxs = a.context_lens;
  auto seg_tiles = [&](int ctx) {  // invalid or empty contexts contribute no tiles
    return (ctx > 0 && ctx <= a.max_context_len) ? (ctx + TK - 1) / TK : 0;
  };

  // ---- total tiles and this wave's share [A, A + n_my)
  int part = 0;
  for (int b = 0; b < S; b += kWave) part += (b + lane < S) ? seg_tiles(ctxs[b + lane]) : 0;
  const int total = wave_sum_int(part) * a.n_units;
  const int W = a.num_waves;
  const int Q = total / W, R = total - (total / W) * W;
  const int A = w * Q + min(w, R);
  const int n_my = Q + (w < R ? 1 : 0);
  if (n_my == 0) return;
  const int A_end = A + n_my;
  auto wave_of = [&](int x) {  // owner of global tile x
    const int cut = R * (Q + 1);
    return x < cut ? x / (Q + 1) : R + (x - cut) / Q;
  };

  // ---- locate tile A: the sequence whose tiles cover it
  int s0 = 0, base = 0;  // base: global index of s0's first tile
  for (int b = 0; b < S; b += kWave) {
    const int ts = ((b + lane < S) ? seg_tiles(ctxs[b + lane]) : 0) * a.n_units;
    const int incl = wave_incl_scan_int(ts, lane);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > A);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      s0 = b + l;
      base += __builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(ts, l);
      break;
    }
    base += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  Cursor cc;  // the tile being computed
  cc.s = s0;
  cc.ctx = ctxs[s0];
  cc.nt = seg_tiles(cc.ctx);
  cc.unit = (A - base) / cc.nt;
  cc.t = (A - base) - cc.unit * cc.nt;
  cc.gstart = base + cc.unit * cc.nt;
  auto advance = [&](Cursor& c) {
    if (++c.t < c.nt) return;
    c.gstart += c.nt;
    c.t = 0;
    if (++c.unit < a.n_units) return;
    c.unit = 0;
    do {
      ++c.s;
      c.ctx = c.s < S ? ctxs[c.s] : 0;
      c.nt = seg_tiles(c.ctx);
    } while (c.nt == 0 && c.s < S);
  };

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
#pragma unroll
    for (int r = 0; r < RK; ++r) {
      const int tok0 = f.t * TK + r * GR;  // first token of the row slot (wave-uniform)
      int p = 0;
      if (real && tok0 < f.ctx) {
        p = trow[tok0 >> a.log2_block];  // scalar load
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
    if (cc.t == 0 && lane == 0)  // this wave starts the segment: record who holds its pieces
      a.seg_desc[cc.s * a.n_units + cc.unit] = make_int2(w, wave_of(cc.gstart + cc.nt - 1));
  };

  // scores, softmax update and P.V for one tile with cn valid tokens
  auto consume = [&](int cn, const u32x4 (&kb)[RK][NL], u32x4 (&vb)[RK][NL]) {
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
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float sc[RK];
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < RK; ++r) {
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < NL; ++j) d = dot16<T>(qv[g][j], kb[r][j], d);
        sc[r] = group_sum<C>(d) * a.scale_log2;
        mt = fmaxf(mt, valid[r] ? sc[r] : -INFINITY);
      }
      const float m_new = fmaxf(m[g], mt);
      // Rescale only when some lane's running max grew; otherwise the factor is
      // exp2(0) = 1 exactly in every lane and skipping it changes nothing.
      if (__builtin_amdgcn_ballot_w64(m_new != m[g]) != 0) {
        const float corr = rescale(m[g], m_new);
        l[g] *= corr;
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[g][e] *= corr;
      }
      m[g] = m_new;
#pragma unroll
      for (int r = 0; r < RK; ++r) {
        const float p = valid[r] ? __builtin_amdgcn_exp2f(sc[r] - m_new) : 0.0f;
        l[g] += p;
        PV<T>::template run<NL>(acc[g], p, vb[r]);
      }
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

  // finish the piece that ends with the current tile: merge the token groups, then
  // write the rows (whole segment) or a piece record (segment shared with other waves)
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
    const bool whole = cc.gstart >= A && cc.gstart + cc.nt <= A_end;
    const bool head = cc.gstart < A;  // the segment began in an earlier wave
    const float qnan = __builtin_nanf("");
    const int64_t row0 = static_cast<int64_t>(cc.s) * a.num_q_heads + h0;
    const int rec = w * 2 + (head ? 0 : 1);
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
          float* dst = a.rec_o + (static_cast<int64_t>(rec) * GT + g) * D + col;
#pragma unroll
          for (int e = 0; e < E; e += 4)
            *reinterpret_cast<u32x4*>(dst + e) = pack16<float>(&o[e]);
        }
      }
      if (!whole && sub == 0) {
        a.rec_m[rec * GT + g] = piece_bad ? qnan : m[g];
        a.rec_l[rec * GT + g] = piece_bad ? qnan : l[g];
      }
    }
  };

  auto process = [&](int i, const u32x4 (&kb)[RK][NL], u32x4 (&vb)[RK][NL], bool stage_bad) {
    if (i == 0 || cc.t == 0) piece_start();
    piece_bad |= stage_bad;
    consume(min(TK, cc.ctx - cc.t * TK), kb, vb);
    if (i == n_my - 1 || cc.t == cc.nt - 1) piece_end();
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
// decode, pass 2: one wave per (sequence, query head).  Empty or invalid contexts get
// their zero or NaN row here; a segment held whole by one wave was written by it; a
// segment split over waves w0..w1 is merged from the tail record of w0 and the head
// records of w0+1..w1, in that order.  Lane p holds piece p's (max, sum); the weights
// go through LDS and each lane sums the pieces' outputs for its dims.
// ---------------------------------------------------------------------------

template <typename T, int D, int GT>
__global__ __launch_bounds__(kWave) void pa_reduce_kernel(
    T* __restrict__ out, const int2* __restrict__ seg_desc, const float* __restrict__ rec_m,
    const float* __restrict__ rec_l, const float* __restrict__ rec_o,
    const int32_t* __restrict__ context_lens, int num_q_heads, int group, int n_gtiles,
    int max_context_len, int w_cap) {
  constexpr int kDPL = D / kWave;  // dims per lane
  __shared__ float s_w[kWave];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  T* dst = out + (static_cast<int64_t>(s) * num_q_heads + h) * D;
  const int ctx = context_lens[s];
  if (ctx <= 0 || ctx > max_context_len) {  // nothing to attend over: zeros; invalid: NaN
    const T fill = static_cast<T>(ctx == 0 ? 0.0f : __builtin_nanf(""));
#pragma unroll
    for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = fill;
    return;
  }
  const int kvh = h / group;
  const int gtile = (h - kvh * group) / GT;
  const int g = h - kvh * group - gtile * GT;
  const int n_units = (num_q_heads / group) * n_gtiles;
  const int2 d = seg_desc[s * n_units + kvh * n_gtiles + gtile];
  if (d.x == d.y) return;  // one wave held the whole segment and wrote the row
  if (d.x < 0 || d.x > d.y || d.y >= w_cap) {  // not written by the stream kernel: no records
#pragma unroll
    for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<T>(__builtin_nanf(""));
    return;
  }
  const int npieces = d.y - d.x + 1;
  auto rec_of = [&](int p) { return p == 0 ? d.x * 2 + 1 : (d.x + p) * 2; };
  float big_m = -INFINITY, den = 0.0f;
  float num[kDPL];
#pragma unroll
  for (int k = 0; k < kDPL; ++k) num[k] = 0.0f;
  for (int p0 = 0; p0 < npieces; p0 += kWave) {
    const int p = p0 + lane;
    const int r = p < npieces ? rec_of(p) * GT + g : 0;
    const float mp = p < npieces ? rec_m[r] : -INFINITY;
    const float lp = p < npieces ? rec_l[r] : 0.0f;
    const float m_new = fmaxf(big_m, wave_max(mp));
    const float c_old = rescale(big_m, m_new);
    const float wp = p < npieces ? lp * __builtin_amdgcn_exp2f(mp - m_new) : 0.0f;
    den = den * c_old + wave_sum(wp);
#pragma unroll
    for (int k = 0; k < kDPL; ++k) num[k] *= c_old;
    __syncthreads();  // the previous group's weights are consumed
    s_w[lane] = wp;
    __syncthreads();
    const int cnt = min(kWave, npieces - p0);
    for (int i = 0; i < cnt; ++i) {
      const float wgt = s_w[i];
      const float* o = rec_o + (static_cast<int64_t>(rec_of(p0 + i)) * GT + g) * D;
#pragma unroll
      for (int k = 0; k < kDPL; ++k) num[k] = fmaf(wgt, o[k * kWave + lane], num[k]);
    }
    big_m = m_new;
  }
#pragma unroll
  for (int k = 0; k < kDPL; ++k) dst[k * kWave + lane] = static_cast<T>(num[k] / den);
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

int group_tile(int group) {  // query heads per wave: 1, 2, 4 or 8 (padded rows are masked)
  return group >= 5 ? 8 : group >= 3 ? 4 : group;
}

// Geometry shared by the size query, the stream launch and the reduce launch.
struct Geom {
  int gt = 1;        // query heads per unit
  int n_gtiles = 1;  // units per kv head
  int n_units = 1;   // segments per sequence
  int w_cap = 1;     // waves the workspace has records for
  size_t desc_bytes = 0, rec_ml_bytes = 0, rec_o_bytes = 0, ws_bytes = 0;
};

// Waves asked for by partition_size > 0: enough that no wave takes much more than
// partition_size tokens of one unit (the batch holds at most S * units * max_ctx).
int64_t waves_for_partition(int64_t num_seqs, int n_units, int max_context_len, int partition_size) {
  if (partition_size <= 0) return 0;
  return (num_seqs * n_units * static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
}

Geom geometry(int64_t num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
              int max_context_len, int partition_size) {
  Geom g;
  const int group = num_q_heads / num_kv_heads;
  g.gt = group_tile(group);
  g.n_gtiles = (group + g.gt - 1) / g.gt;
  g.n_units = num_kv_heads * g.n_gtiles;
  int64_t w = kMaxWaves;
  const int64_t want = waves_for_partition(num_seqs, g.n_units, max_context_len, partition_size);
  if (want > w) w = want;
  g.w_cap = static_cast<int>(w > (1 << 28) ? (1 << 28) : w);
  g.desc_bytes = align256(static_cast<size_t>(num_seqs) * g.n_units * 2 * sizeof(int));
  g.rec_ml_bytes = align256(static_cast<size_t>(2) * g.w_cap * g.gt * sizeof(float));
  g.rec_o_bytes = align256(static_cast<size_t>(2) * g.w_cap * g.gt * head_dim * sizeof(float));
  g.ws_bytes = g.desc_bytes + 2 * g.rec_ml_bytes + g.rec_o_bytes;
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
};

int check_decode(const DecodeCall& c, Geom* g) {
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
  if (c.num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d > 65535", c.num_seqs);
  *g = geometry(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim, c.max_context_len, c.partition_size);
  // tile counts are 32-bit in the kernel (a tile holds at least 8 tokens)
  if (static_cast<int64_t>(c.num_seqs) * g->n_units * ((static_cast<int64_t>(c.max_context_len) + 7) / 8) >
      (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "batch too large: more than 2^31 - 1 tiles");
  if (c.num_blocks > (static_cast<int64_t>(1) << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "num_blocks above 2^31 - 1");
  if (static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim * (c.dtype == PA_F16 ? 2 : 4) >
      (static_cast<int64_t>(1) << 32) - 1)
    return fail(PA_ERR_INVALID_ARG, "one block of one layer exceeds 4 GiB");
  if (c.num_seqs == 0) return PA_OK;
  if (!c.out || !c.q || !c.k_cache || !c.v_cache || !c.block_tables || !c.context_lens)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(c.out, 16) || !aligned(c.q, 16) || !aligned(c.k_cache, 16) || !aligned(c.v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "out, q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(c.block_tables, 4) || !aligned(c.context_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables and context_lens must be 4-byte aligned");
  if (!c.workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", g->ws_bytes);
  if (c.workspace_bytes < g->ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", c.workspace_bytes, g->ws_bytes);
  if (!aligned(c.workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
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
  p.rec_m = reinterpret_cast<float*>(b + g.desc_bytes);
  p.rec_l = reinterpret_cast<float*>(b + g.desc_bytes + g.rec_ml_bytes);
  p.rec_o = reinterpret_cast<float*>(b + g.desc_bytes + 2 * g.rec_ml_bytes);
  return p;
}

// Resident one-wave work-groups of a kernel on the current device (cached per device
// and kernel; the answer is fixed for a given build and device).
template <typename T, int D, int GT>
int resident_waves() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return kMaxWaves;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pa_stream_kernel<T, D, GT>, kWave, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu <= 0 || cus <= 0) {
      (void)hipGetLastError();
      return kMaxWaves;
    }
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

// Waves of one launch: the resident count (at most kMaxWaves), raised with
// partition_size > 0; never more than the workspace has records for.
template <typename T, int D, int GT>
int waves_for(const DecodeCall& c, const Geom& g) {
  int64_t w = resident_waves<T, D, GT>();
  if (w > kMaxWaves) w = kMaxWaves;
  const int64_t want = waves_for_partition(c.num_seqs, g.n_units, c.max_context_len, c.partition_size);
  if (want > w) w = want;
  if (w > g.w_cap) w = g.w_cap;
  return static_cast<int>(w < 1 ? 1 : w);
}

template <typename T, int D, int GT>
int launch_stream(const DecodeCall& c, const Geom& g) {
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
  a.scale_log2 = static_cast<float>(static_cast<double>(c.scale) * 1.4426950408889634);
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
  a.num_waves = waves_for<T, D, GT>(c, g);
  hipLaunchKernelGGL((pa_stream_kernel<T, D, GT>), dim3(a.num_waves), dim3(kWave), 0, c.stream, a);
  return check_hip("pa_stream_kernel launch");
}

template <typename T, int D, int GT>
int launch_reduce(const DecodeCall& c, const Geom& g) {
  const WsParts ws = split_workspace(c.workspace, g);
  hipLaunchKernelGGL((pa_reduce_kernel<T, D, GT>), dim3(c.num_q_heads, c.num_seqs), dim3(kWave), 0,
                     c.stream, static_cast<T*>(c.out), ws.desc, ws.rec_m, ws.rec_l, ws.rec_o,
                     c.context_lens, c.num_q_heads, c.num_q_heads / c.num_kv_heads, g.n_gtiles,
                     c.max_context_len, g.w_cap);
  return check_hip("pa_reduce_kernel launch");
}

template <int Which, typename T, int D>
int dispatch_gt(const DecodeCall& c, const Geom& g) {
  switch (g.gt) {
    case 1: return Which == 0 ? launch_stream<T, D, 1>(c, g) : launch_reduce<T, D, 1>(c, g);
    case 2: return Which == 0 ? launch_stream<T, D, 2>(c, g) : launch_reduce<T, D, 2>(c, g);
    case 4: return Which == 0 ? launch_stream<T, D, 4>(c, g) : launch_reduce<T, D, 4>(c, g);
    default: return Which == 0 ? launch_stream<T, D, 8>(c, g) : launch_reduce<T, D, 8>(c, g);
  }
}

// Which = 0: the stream kernel; 1: the reduce kernel
template <int Which>
int dispatch(const DecodeCall& c, const Geom& g) {
  if (c.num_seqs == 0) return PA_OK;
  if (c.dtype == PA_F16)
    return c.head_dim == 64 ? dispatch_gt<Which, f16, 64>(c, g) : dispatch_gt<Which, f16, 128>(c, g);
  return c.head_dim == 64 ? dispatch_gt<Which, float, 64>(c, g) : dispatch_gt<Which, float, 128>(c, g);
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

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || partition_size < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  return geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size).ws_bytes;
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
  if (num_seqs == 0) return PA_OK;
  const Geom g = geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size);
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

}  // extern "C"
