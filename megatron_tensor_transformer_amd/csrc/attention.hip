// Core of the tensor-parallel self-attention shard: per (shard, batch entry,
// head), S = q·kᵀ/√dh with an optional causal mask and an optional general
// mask, A = softmax(S) row by row, o = A·v ([TRAIN] Attention 层 section; the
// causal mask is the implicit one of [EFF] §4.2's fused softmax, the general
// one that section's other kernel, e.g. BERT's padding mask), and its backward
//   dv = Aᵀ·do,  dS = A ⊙ (do·vᵀ − δ),  δ_i = Σ_j A_ij (do_i·v_j) = do_i·o_i,
//   dq = dS·k/√dh,  dk = dSᵀ·q/√dh.
// The heads of a shard are the contiguous column groups of the column-parallel
// QKV output ([SENSE] §2.1.1, multi-head attention module: per-head (q, k, v)
// columns); tokens are rows in [s, b] order ([EFF] §4.2 layout).
//
// Layouts (T = resident shards, n = s·b, row r = s_idx·b + b_idx):
//   qkv [T][n][nh·3·dh]: head h's q, k, v at columns h·3dh + {0, dh, 2dh}
//   o   [T][n][nh·dh]:   head h at columns h·dh (the row-parallel input)
//   lse [T][b][nh][s]:   natural log of Σ_j exp(S_ij) per query row (fp32)
//
// bf16 path: a flash-attention forward on the matrix cores.  A 256-thread
// workgroup takes 128 query rows of one (shard, batch entry, head), 32 per
// wave, with the wave's q fragments in registers; 64-row K and V tiles are
// streamed into LDS with buffer→LDS DMA, double-buffered.  Per tile a wave
// computes Sᵀ = K·Qᵀ so that each lane holds logits of its own query row
// (lane L: row L%32), keeps the running row maximum and sum (online softmax,
// base-2 exponentials with log2(e)/√dh folded into one fma), and accumulates
// Oᵀ = Vᵀ·Pᵀ, again with row L%32 in lane L, so the rescaling by the running
// maximum is lane-local.  The MFMA's k order for Pᵀ is a permutation of the
// tile's keys (the one the S accumulators already hold); the V fragments are
// read with the same permutation through the transposing LDS read, so no
// register shuffle is needed.
//
// LDS fragment reads are explicit inline asm, issued ahead of their MFMAs and
// waited for with counted waits; one barrier per key (or query) tile.  A
// general mask arrives bit-packed once per batch (by query row for the
// forward and dq, by key column for dk/dv); a lane reads one word per 32
// positions a tile ahead, and a wave skips tiles it cannot see at all.
//
// fp32 path (the numeric-alignment path, not tuned): two lanes per query row
// (forward, dq) or key row (dk, dv), each holding half of the row's columns;
// online softmax in fp32.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tile_map.h"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float RESCALE = 8.f;  // exp2 units the running maximum may pass before o is rescaled
constexpr int AQ = 128;   // query (key) rows per workgroup (4 waves × 32)
constexpr int AKV = 64;   // key rows per step
constexpr int ATHR = 256;
constexpr uint32_t AOOB = 0x80000000u;

// Byte offset of 16-B chunk `chunk` of row `row` in a [AKV][DH] bf16 tile.
// The XOR swizzle keeps both the 16-row column reads (ds_read_b128, one chunk
// of 16 consecutive rows) and the transposing reads (4 consecutive rows × 4
// consecutive chunks) free of bank conflicts.
template <int DH>
__device__ __forceinline__ uint32_t kv_slot(int row, int chunk) {
  int f;
  if constexpr (DH == 128) f = ((row & 3) << 2) | ((row >> 2) & 3);
  else f = (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  return static_cast<uint32_t>(row * (DH * 2) + ((chunk ^ f) << 4));
}

// The general mask arrives bit-packed (tpmlp_attn_pack_mask): W = ⌈s/32⌉
// 32-bit words per position, part 0 by query row (bit j of word w of row q:
// key 32w + j hidden from q), part 1 by key column (bit i of word w of column
// k: k hidden from query 32w + i); positions past s are set.  A lane reads one
// word per 32-wide half tile through a buffer resource.
__device__ uint32_t tpmlp_llvm_buffer_load_u32(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.i32");
__device__ i32x4 tpmlp_llvm_buffer_load_v4(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4i32");

// The 16 bits of a 32-position mask word that belong to this lane's
// accumulator entries: entry v = 4g + e is position 8g + 4·hi + e.
__device__ __forceinline__ uint32_t lane_bits16(uint32_t word, int hi) {
  const uint32_t x = (word >> (4 * hi)) & 0x0F0F0F0Fu;
  return (x & 0xFu) | ((x >> 4) & 0xF0u) | ((x >> 8) & 0xF00u) | ((x >> 12) & 0xF000u);
}

// −∞ where bit v of bits is set (the general mask hides accumulator entry v).
__device__ __forceinline__ void apply_mask16(f32x16& x, uint32_t bits) {
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if ((bits >> v) & 1u) x[v] = -INFINITY;
}

struct AttnArgs {
  const void* qkv;
  void* o;
  float* lse;
  int s, b, nh, T;
  int nqb;            // query blocks of AQ rows per (shard, batch entry, head)
  float scale;        // 1/√dh
  float scale_log2;   // log2(e)/√dh
  uint32_t qkv_shard_bytes;
  const uint32_t* mask;  // packed general mask (2 parts of [b][s][mw] words), or null
  int mw;                // words per position, ⌈s/32⌉
};

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
// Workgroup -> (shard, batch entry, head) and block position p (0 = the most
// work): each XCD keeps the blocks of a contiguous run of heads (shared K/V or
// Q/dO panels in its L2).  Causal blocks differ in length, so heavy_first_block
// starts all the run's longest blocks first and the short ones fill in behind
// them; without the causal mask they are alike and go head by head (a head's
// blocks run together and share its panel while it is in the L2).
template <bool CAUSAL>
__device__ __forceinline__ void attn_block_at(int nh, int b, int nblk, int G, int wg, int& T, int& bi, int& h, int& p) {
  int flat;
  if constexpr (CAUSAL) {
    heavy_first_block(G / nblk, nblk, wg, flat, p);
  } else {
    int begin, count;
    xcd_range(G, wg & 7, begin, count);
    const int x = begin + (wg >> 3);
    flat = x / nblk;
    p = x - flat * nblk;
  }
  h = flat % nh;
  flat /= nh;
  bi = flat % b;
  T = flat / b;
}
template <bool CAUSAL>
__device__ __forceinline__ void attn_block(int nh, int b, int nblk, int& T, int& bi, int& h, int& p) {
  attn_block_at<CAUSAL>(nh, b, nblk, static_cast<int>(gridDim.x), static_cast<int>(blockIdx.x), T, bi, h, p);
}

// Forward: the longest causal query blocks are the last in the sequence.
template <bool CAUSAL>
__device__ __forceinline__ void attn_coords(const AttnArgs& a, int& T, int& bi, int& h, int& qb) {
  int p;
  attn_block<CAUSAL>(a.nh, a.b, a.nqb, T, bi, h, p);
  qb = a.nqb - 1 - p;
}

// DMA of one [AKV][DH] tile: rows j·AKV .. +63 of a token-major tensor whose
// row r (sequence position) of batch entry bi starts at element
// (r·b + bi)·row_len, columns col .. col+DH-1.  Rows past s are zero-filled
// (an offset past the descriptor's range).
template <int DH>
__device__ __forceinline__ void load_tile(i32x4 rsrc, TPMLP_LDS char* tile, int s, int b, int bi, int64_t row_len,
                                          int64_t col, int j, int wave, int lane) {
  constexpr int NI = AKV * DH * 2 / 1024 / 4;   // 1-KiB DMA loads per wave
  constexpr int RPI = 1024 / (DH * 2);          // rows per load
  constexpr int CPR = DH / 8;                   // chunks per row
  // the LDS destination (M0) from a scalar copy of the uniform wave index
  const int ws = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int I = wave * NI + q;
    const int row = I * RPI + lane / CPR;
    const int slot = lane % CPR;
    int f;
    if constexpr (DH == 128) f = ((row & 3) << 2) | ((row >> 2) & 3);
    else f = (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    const int chunk = slot ^ f;
    const int r = j * AKV + row;
    const uint32_t voff =
        r < s ? static_cast<uint32_t>(((static_cast<int64_t>(r) * b + bi) * row_len + col + chunk * 8) * 2) : AOOB;
    buffer_load_lds16(rsrc, tile + (ws * NI + q) * 1024, voff);
  }
}

// Workgroup barrier that is also a compiler barrier for memory accesses (LDS
// reads must not move above it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// values 8·c2 .. 8·c2+7 of an accumulator block as a bf16 MFMA operand
__device__ __forceinline__ bf16x8 pack_acc(const f32x16& x, int c2) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = f2bf(x[8 * c2 + e]);
  return f;
}

// max / sum of a value over lanes L and L^32 (the two halves of a row):
// v_permlane32_swap gives each lane both halves' values, in a VALU op.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keep entries (u, v) of a tile's accumulator pair whose index
// 32u + 8(v/4) + 4·hi + v%4 (relative to the tile) lies in [lo, hi_): the
// rest become `fill`.  lo and hi_ are per-lane bounds already relative to the
// tile and to this lane's 4·hi offset.
__device__ __forceinline__ void mask_range(f32x16 (&x)[2], int lo, int hi_, float fill) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = 32 * u + 8 * (v >> 2) + (v & 3);
      x[u][v] = (k >= lo && k < hi_) ? x[u][v] : fill;
    }
}

// the same for one accumulator block u
__device__ __forceinline__ void mask_range1(f32x16& x, int u, int lo, int hi_, float fill) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int k = 32 * u + 8 * (v >> 2) + (v & 3);
    x[v] = (k >= lo && k < hi_) ? x[v] : fill;
  }
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-lane DMA plan of a [AKV][DH] tile: the byte offset of this lane's 16-B
// chunk for key block 0 and its row; block j adds j·AKV rows.
template <int DH, int NW = 4>
struct TilePlan {
  static constexpr int NI = AKV * DH * 2 / 1024 / NW;
  uint32_t voff[NI];
  int row[NI];
};

template <int DH, int NW = 4>
__device__ __forceinline__ TilePlan<DH, NW> tile_plan(int b, int bi, int64_t row_len, int64_t col, int wave,
                                                      int lane) {
  constexpr int RPI = 1024 / (DH * 2), CPR = DH / 8;
  TilePlan<DH, NW> p;
#pragma unroll
  for (int q = 0; q < TilePlan<DH, NW>::NI; ++q) {
    const int I = wave * TilePlan<DH, NW>::NI + q;
    const int row = I * RPI + lane / CPR;
    int f;
    if constexpr (DH == 128) f = ((row & 3) << 2) | ((row >> 2) & 3);
    else f = (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    const int chunk = (lane % CPR) ^ f;
    p.row[q] = row;
    p.voff[q] = static_cast<uint32_t>(((static_cast<int64_t>(row) * b + bi) * row_len + col + chunk * 8) * 2);
  }
  return p;
}

// DMA of key/query block j by plan p into `tile` (stride = bytes per AKV rows
// of the tensor, rows past s zero-filled).
template <int DH, int NW = 4>
__device__ __forceinline__ void issue_tile(i32x4 rsrc, TPMLP_LDS char* tile, const TilePlan<DH, NW>& p, int j,
                                           uint32_t stride, int s, int wave) {
  const uint32_t jo = static_cast<uint32_t>(j) * stride;
  const int ws = __builtin_amdgcn_readfirstlane(wave);  // scalar LDS destinations (M0)
  if (j * AKV + AKV <= s) {  // the whole block is in range: no per-row check
#pragma unroll
    for (int q = 0; q < TilePlan<DH, NW>::NI; ++q)
      buffer_load_lds16(rsrc, tile + (ws * TilePlan<DH, NW>::NI + q) * 1024, p.voff[q] + jo);
  } else {
#pragma unroll
    for (int q = 0; q < TilePlan<DH, NW>::NI; ++q) {
      const uint32_t voff = j * AKV + p.row[q] < s ? p.voff[q] + jo : AOOB;
      buffer_load_lds16(rsrc, tile + (ws * TilePlan<DH, NW>::NI + q) * 1024, voff);
    }
  }
}

// Per-lane LDS addresses of the transposing reads of a tile at its base
// (blocks (u, c2) add (32u + 16c2) rows, a constant: the swizzle depends on
// the row modulo 16 only).  Entry 2d + k: column block d, second read k.
template <int DH, int ND>
__device__ __forceinline__ void tr_addrs(uint32_t base, int lane, uint32_t (&o)[2 * ND]) {
  const int g = lane >> 4, i = lane & 15;
  const int r = 4 * (lane >> 5) + (i >> 2);
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const int col = 32 * d + 16 * (g & 1) + 4 * (i & 3);
    o[2 * d] = base + kv_slot<DH>(r, col >> 3) + (col & 7) * 2;
    o[2 * d + 1] = base + kv_slot<DH>(r + 8, col >> 3) + (col & 7) * 2;
  }
}

// Transposed MFMA operands of one 16-row block at byte offset IMM (stage,
// tile and block) from the per-lane addresses of tr_addrs: lane L gets
// columns 32d + L%32 (d < ND), rows 4·(L/32) + {0..3} then the same + 8, the
// accumulators' key order.  Software-pipelined in three parts: tr_issue
// sends the 2·ND reads of a block (no wait), tr_wait<N> waits until at most N
// newer LDS operations are in flight (LDS completes in order, so every read
// issued before those N is done; other LDS operations only make the wait more
// conservative), and tr_frags assembles the operands.  The reads are inline
// asm: the transposing-read builtin made the compiler wait for every
// outstanding buffer→LDS load before it, and its element-wise assembly into
// bf16x8 was miscompiled (only the first dword survived).  The offset field
// has 16 bits: a larger IMM moves its high part into the address.
template <int DH, int ND, int IMM>
__device__ __forceinline__ void tr_issue(const uint32_t (&ad)[2 * ND], i32x2 (&t)[2 * ND]) {
  constexpr uint32_t HI = (static_cast<uint32_t>(IMM) >> 16) << 16, LO = IMM - HI;
#pragma unroll
  for (int k = 0; k < 2 * ND; ++k)
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(t[k]) : "v"(ad[k] + HI), "i"(LO) : "memory");
}

template <int N, int ND>
__device__ __forceinline__ void tr_wait(i32x2 (&t)[2 * ND]) {
  static_assert(N == 0 || N == 4 || N == 8, "lgkmcnt");
  if constexpr (N == 8) asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(t[0])::"memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(t[0])::"memory");
  else asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(t[0])::"memory");
#pragma unroll
  for (int k = 1; k < 2 * ND; ++k) asm volatile("" : "+v"(t[k]));
}

template <int ND>
__device__ __forceinline__ void tr_frags(const i32x2 (&t)[2 * ND], bf16x8 (&out)[ND]) {
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    i32x4 w;
    w[0] = t[2 * d][0];
    w[1] = t[2 * d][1];
    w[2] = t[2 * d + 1][0];
    w[3] = t[2 * d + 1][1];
    out[d] = __builtin_bit_cast(bf16x8, w);
  }
}

template <int V>
using ic = std::integral_constant<int, V>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>{});
    static_for<I + 1, N>(f);
  }
}

// ds_read_b128 at addr + IMM, issued now; the result may be used only after
// an lgkm_wait that covers it.
template <int IMM>
__device__ __forceinline__ i32x4 lds_rd128(uint32_t addr) {
  static_assert(IMM >= 0 && IMM < 65536, "ds offset");
  i32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(IMM) : "memory");
  return r;
}

// Wait until at most N LDS reads are in flight, and publish x and y (two
// results of reads issued before those N) to the compiler.
template <int N>
__device__ __forceinline__ void lgkm_wait(i32x4& x, i32x4& y) {
  static_assert(N == 0 || N == 2 || N == 4, "lgkmcnt");
  if constexpr (N == 4) asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(x), "+v"(y)::"memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(x), "+v"(y)::"memory");
  else asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x), "+v"(y)::"memory");
}

// Writes a wave's 32×DH result block, held as 32-row MFMA accumulators (lane
// L: row L%32, columns 32d + 8(v/4) + 4·(L/32) + v%4), times `scale`, as bf16
// rows dst + r·ld for r < nrows.  Stored directly, each 8-B piece would make a
// store touch 32 rows; instead the wave stages the block in its own LDS region
// `reg` (32·DH·2 bytes) and writes whole rows, 16 B per lane.  Staging layout:
// 8-B unit k of row r at unit k ^ g(r), g(r) = r (dh 128) or r / 2 (dh 64), so
// the 32 lanes of each half-wave write 32 distinct bank pairs; a 16-B read of
// units 2m, 2m+1 finds them in one aligned slot, swapped when g(r) is odd.
template <int DH>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[DH / 32], float scale, uint32_t reg,
                                                  bf16* dst, int64_t ld, int nrows, int lane) {
  constexpr int RB = DH * 2, GS = DH == 128 ? 0 : 1;
  constexpr int CPR = DH / 8, RPI = 64 / CPR, NS = 32 / RPI;  // 16-B chunks per row, rows per store
  const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int d = 0; d < DH / 32; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = f2bf(acc[d][4 * q4 + e] * scale);
      const uint32_t ad = reg + r32 * RB + (((2 * (4 * d + q4) + hi) ^ (r32 >> GS)) << 3);
      asm volatile("ds_write_b64 %0, %1" ::"v"(ad), "v"(__builtin_bit_cast(i32x2, w)) : "memory");
    }
  lds_wait();
  const int mc = lane % CPR;
  i32x4 v[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int R = i * RPI + lane / CPR;
    v[i] = lds_rd128<0>(reg + R * RB + (((2 * mc) ^ (R >> GS)) & ~1) * 8);
  }
  lds_wait();
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    asm volatile("" : "+v"(v[i]));
    const int R = i * RPI + lane / CPR;
    if ((R >> GS) & 1) v[i] = i32x4{v[i][2], v[i][3], v[i][0], v[i][1]};
    if (R < nrows) *reinterpret_cast<i32x4*>(dst + R * ld + 8 * mc) = v[i];
  }
}

template <int DH, bool CAUSAL, bool GMASK>
__global__ __launch_bounds__(ATHR, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int TILE = AKV * DH * 2, RB = DH * 2;
  constexpr int NC = DH / 16;   // k16 slices of the head dimension
  constexpr int ND = DH / 32;   // 32-wide head-dimension blocks of o
  constexpr int NW = ATHR / 64;
  constexpr int NI = TilePlan<DH, NW>::NI;
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE];
  TPMLP_LDS char* lds = (TPMLP_LDS char*)(smem);
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  int T, bi, h, qb;
  attn_coords<CAUSAL>(a, T, bi, h, qb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * AQ + wave * 32;
  const int qrow = q0 + r32;
  // this batch entry's general mask (read only when GMASK)
  const i32x4 mrs = GMASK ? make_rsrc(a.mask + static_cast<int64_t>(bi) * a.s * a.mw,
                                        static_cast<uint32_t>(static_cast<int64_t>(a.s) * a.mw * 4))
                             : i32x4{0, 0, 0, 0};
  const int64_t row_len = static_cast<int64_t>(a.nh) * 3 * DH;
  const bf16* qkv = static_cast<const bf16*>(a.qkv) + static_cast<int64_t>(T) * a.s * a.b * row_len;
  const i32x4 rsrc = make_rsrc(qkv, a.qkv_shard_bytes);
  const uint32_t stride = static_cast<uint32_t>(static_cast<int64_t>(AKV) * a.b * row_len * 2);

  // key blocks this workgroup visits
  const int kv_end = CAUSAL ? min(a.s, qb * AQ + AQ) : a.s;
  const int nkv = (kv_end + AKV - 1) / AKV;

  const int64_t kcol = static_cast<int64_t>(h) * 3 * DH + DH;
  const TilePlan<DH, NW> kp = tile_plan<DH, NW>(a.b, bi, row_len, kcol, wave, lane);
  const TilePlan<DH, NW> vp = tile_plan<DH, NW>(a.b, bi, row_len, kcol + DH, wave, lane);
  // prologue: K and V of block 0 into stage 0, and the workgroup's 128 query
  // rows (two 64-row tiles, rows past s zero-filled) into stage 1, which is
  // free until the first step's barrier: whole rows per DMA load, where each
  // lane loading its own fragments would touch 32 rows per load
  issue_tile<DH, NW>(rsrc, lds, kp, 0, stride, a.s, wave);
  issue_tile<DH, NW>(rsrc, lds + TILE, vp, 0, stride, a.s, wave);
  {
    const TilePlan<DH, NW> qp = tile_plan<DH, NW>(a.b, bi, row_len, static_cast<int64_t>(h) * 3 * DH, wave, lane);
    issue_tile<DH, NW>(rsrc, lds + 2 * TILE, qp, 2 * qb, stride, a.s, wave);
    issue_tile<DH, NW>(rsrc, lds + 3 * TILE, qp, 2 * qb + 1, stride, a.s, wave);
  }
  // row-fragment offsets (row r32, chunk 2c + hi) and transposed-read addresses
  uint32_t ko[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) ko[c] = lds_base + kv_slot<DH>(r32, 2 * c + hi);

  // this lane's q fragments: row qrow, dh = 16c + 8·hi + 0..7 (the wave's 32
  // rows are rows 32·(wave % 2) .. of query tile wave / 2)
  bf16x8 qf[NC];
  {
    wait_vmcnt<0>();
    lds_barrier();
    const uint32_t qoff = 2 * TILE + (wave >> 1) * TILE + (wave & 1) * 32 * RB;
    i32x4 qr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) qr[c] = lds_rd128<0>(ko[c] + qoff);
    lds_wait();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      asm volatile("" : "+v"(qr[c]));
      qf[c] = __builtin_bit_cast(bf16x8, qr[c]);
    }
  }
  uint32_t va[2 * ND];
  tr_addrs<DH, ND>(lds_base, lane, va);

  f32x16 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.f;
  float m = -INFINITY, l = 0.f;

  // general-mask words of key tile jj for this lane's row (one per 32 keys)
  uint32_t mwn[2] = {~0u, ~0u};
  auto mask_words = [&](int jj) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pos = jj * AKV + 32 * u;
      mwn[u] = qrow < a.s && pos < a.s ? tpmlp_llvm_buffer_load_u32(mrs, (qrow * a.mw + pos / 32) * 4, 0, 0) : ~0u;
    }
  };
  if constexpr (GMASK) mask_words(0);

  // one key tile in stage ST (compile-time, so every LDS offset is an
  // immediate).  One barrier per tile: after it every wave has finished the
  // previous tile, so the other stage is free and the next tile's DMA is
  // issued into it, running during this tile.
  auto step = [&](auto stc, int j) {
    constexpr int ST = decltype(stc)::value;
    wait_vmcnt<0>();  // this wave's share of tile j (the only DMA in flight)
    lds_barrier();
    // A causal tile whose first key is past the wave's last query row (or a
    // wave wholly past s) contributes nothing: its work is skipped.
    const int t0 = j * AKV;
    const bool dead = q0 >= a.s || (CAUSAL && t0 > q0 + 31);
    // general mask of the tile's keys for this lane's row (bit v of mk[u]:
    // accumulator entry v of half u), from the words loaded one tile ahead;
    // the next tile's words are loaded before its DMA
    uint32_t mk[2] = {0u, 0u};
    bool hidden = false;
    if constexpr (GMASK) {
      mk[0] = lane_bits16(mwn[0], hi);
      mk[1] = lane_bits16(mwn[1], hi);
      if (j + 1 < nkv) mask_words(j + 1);
      hidden = __all((mk[0] & mk[1]) == 0xFFFFu);  // the wave sees no key of the tile
    }
    if (j + 1 < nkv) {
      TPMLP_LDS char* nxt = lds + (ST ^ 1) * 2 * TILE;
      issue_tile<DH, NW>(rsrc, nxt, kp, j + 1, stride, a.s, wave);
      issue_tile<DH, NW>(rsrc, nxt + TILE, vp, j + 1, stride, a.s, wave);
    }
    if (dead || hidden) return;

    // Sᵀ block: sacc[u][v] = S[qrow][kv], kv = 64j + 32u + 8(v/4) + 4·hi + v%4.
    // The two 32-key halves alternate (independent accumulators), and the K
    // fragments of slice c + 3 are read while slice c's MFMAs run (four
    // register pairs in a ring).
    constexpr int KB = ST * 2 * TILE;
    f32x16 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[u][v] = 0.f;
    i32x4 kr[4][2];
    auto kread = [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      kr[c % 4][0] = lds_rd128<KB>(ko[c]);
      kr[c % 4][1] = lds_rd128<KB + 32 * RB>(ko[c]);
    };
    static_for<0, (NC < 3 ? NC : 3)>(kread);
    static_for<0, NC>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      constexpr int later = 2 * (NC - 1 - c < 2 ? NC - 1 - c : 2);  // reads issued after slice c's
      lgkm_wait<later>(kr[c % 4][0], kr[c % 4][1]);
      sacc[0] = mfma(__builtin_bit_cast(bf16x8, kr[c % 4][0]), qf[c], sacc[0]);
      sacc[1] = mfma(__builtin_bit_cast(bf16x8, kr[c % 4][1]), qf[c], sacc[1]);
      if constexpr (c + 3 < NC) kread(ic<c + 3>{});
    });

    // mask (only tiles that reach past s or, causal, past the wave's first
    // query row), running maximum, exponentials, running sum
    if (t0 + AKV > a.s || (CAUSAL && t0 + AKV - 1 > q0)) {
      const int lim = CAUSAL ? min(qrow + 1, a.s) : a.s;
      mask_range(sacc, -1 << 30, lim - t0 - 4 * hi, -INFINITY);
    }
    if constexpr (GMASK) {
      apply_mask16(sacc[0], mk[0]);
      apply_mask16(sacc[1], mk[1]);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sacc[u][v]);
    mloc = pair_max(mloc);
    // The exponent reference m moves only when some row's maximum passes it
    // by more than RESCALE in exp2 units (always on the first tile, where m is
    // −∞).  Otherwise P = 2^((S−m)·log2(e)/√dh) stays ≤ 2^RESCALE, and
    // o = Σ P·v / Σ P and lse = m/√dh + ln Σ P hold for any reference, so the
    // rescaling of the running sum and of o is skipped.
    const float mnew = fmaxf(m, mloc);
    if (__any((mnew - m) * a.scale_log2 > RESCALE)) {
      const float alpha = __builtin_amdgcn_exp2f((m - (mnew == -INFINITY ? 0.f : mnew)) * a.scale_log2);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[d][v] *= alpha;
      m = mnew;
    }
    const float off = -(m == -INFINITY ? 0.f : m) * a.scale_log2;
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[u][v], a.scale_log2, off));
        sacc[u][v] = p;
        lsum += p;
      }
    l += pair_sum(lsum);

    // Oᵀ += Vᵀ·Pᵀ over the tile's keys, 16 at a time.  P fragment (u, c2):
    // this lane's values v = 8·c2 .. 8·c2+7 of sacc[u]; they are keys
    // 32u + 16c2 + {0..3, 8..11} (hi = 0) or {4..7, 12..15} (hi = 1), and the
    // V fragment rows are read in that same order.
    // The reads of block g+1 are in flight while block g's MFMAs run (two
    // register sets; a set is refilled only after the MFMAs that read it
    // were issued).
    constexpr int VB = ST * 2 * TILE + TILE;
    constexpr int NR = 2 * ND;
    i32x2 ta[NR], tb[NR];
    bf16x8 vf[ND];
    tr_issue<DH, ND, VB>(va, ta);
    tr_issue<DH, ND, VB + 16 * RB>(va, tb);
    tr_wait<NR, ND>(ta);
    tr_frags<ND>(ta, vf);
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = mfma(vf[d], pack_acc(sacc[0], 0), oacc[d]);
    asm volatile("s_nop 1" ::: "memory");
    tr_issue<DH, ND, VB + 32 * RB>(va, ta);
    tr_wait<NR, ND>(tb);
    tr_frags<ND>(tb, vf);
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = mfma(vf[d], pack_acc(sacc[0], 1), oacc[d]);
    asm volatile("s_nop 1" ::: "memory");
    tr_issue<DH, ND, VB + 48 * RB>(va, tb);
    tr_wait<NR, ND>(ta);
    tr_frags<ND>(ta, vf);
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = mfma(vf[d], pack_acc(sacc[1], 0), oacc[d]);
    tr_wait<0, ND>(tb);
    tr_frags<ND>(tb, vf);
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = mfma(vf[d], pack_acc(sacc[1], 1), oacc[d]);
  };
  int j = 0;
  for (; j + 1 < nkv; j += 2) {
    step(ic<0>{}, j);
    step(ic<1>{}, j + 1);
  }
  if (j < nkv) step(ic<0>{}, j);

  // o = oacc / l, staged through the stage the last tile did not use (free
  // since that tile's barrier: every wave had finished the tile before it,
  // and no DMA went into it after), one 32-row region per wave
  {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    bf16* ob = static_cast<bf16*>(a.o) + static_cast<int64_t>(T) * a.s * a.b * a.nh * DH +
               (static_cast<int64_t>(q0) * a.b + bi) * a.nh * DH + h * DH;
    store_rows_staged<DH>(oacc, inv, lds_base + (nkv & 1) * 2 * TILE + wave * 32 * RB, ob,
                          static_cast<int64_t>(a.b) * a.nh * DH, a.s - q0, lane);
  }
  if (qrow < a.s && hi == 0) {
    const float lse = l > 0.f ? m * a.scale + logf(l) : -INFINITY;
    a.lse[((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s + qrow] = lse;
  }
}

// ------------------------------------------------------------------ fp32 path
// Two lanes per query row of one (shard, batch entry, head): lane half j of a
// pair holds columns j·dh/2 .. of the row (q, the o accumulator), and the dot
// products are the two halves' partial sums added across the pair.
template <int DH>
__device__ __forceinline__ float pair_dot_sum(float x) {
  return x + __shfl_xor(x, 1);
}

template <int DH, bool CAUSAL>
__global__ __launch_bounds__(128) void attn_fwd_f32_kernel(AttnArgs a) {
  constexpr int H = DH / 2;
  const int64_t idx = (static_cast<int64_t>(blockIdx.x) * 128 + threadIdx.x) >> 1;
  const int j = threadIdx.x & 1;
  const int64_t total = static_cast<int64_t>(a.T) * a.b * a.nh * a.s;
  if (idx >= total) return;  // both lanes of a pair leave together
  const int q = static_cast<int>(idx % a.s);
  int64_t r = idx / a.s;
  const int h = static_cast<int>(r % a.nh);
  r /= a.nh;
  const int bi = static_cast<int>(r % a.b);
  const int T = static_cast<int>(r / a.b);
  const int64_t row_len = static_cast<int64_t>(a.nh) * 3 * DH;
  const float* qkv = static_cast<const float*>(a.qkv) + static_cast<int64_t>(T) * a.s * a.b * row_len;
  const float* qp = qkv + (static_cast<int64_t>(q) * a.b + bi) * row_len + h * 3 * DH + j * H;
  float qv[H], acc[H];
#pragma unroll
  for (int d = 0; d < H; ++d) {
    qv[d] = qp[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = CAUSAL ? q + 1 : a.s;
  const uint32_t* mrow = a.mask ? a.mask + (static_cast<int64_t>(bi) * a.s + q) * a.mw : nullptr;
  for (int kv = 0; kv < kend; ++kv) {
    if (mrow && ((mrow[kv >> 5] >> (kv & 31)) & 1u)) continue;  // the same for both lanes
    const float* kp = qkv + (static_cast<int64_t>(kv) * a.b + bi) * row_len + h * 3 * DH + DH + j * H;
    float sdot = 0.f;
#pragma unroll
    for (int d = 0; d < H; ++d) sdot = fmaf(qv[d], kp[d], sdot);
    const float sv = pair_dot_sum<DH>(sdot) * a.scale;
    const float mn = fmaxf(m, sv);
    const float alpha = expf(m - mn), p = expf(sv - mn);
    l = l * alpha + p;
#pragma unroll
    for (int d = 0; d < H; ++d) acc[d] = fmaf(p, kp[DH + d], acc[d] * alpha);
    m = mn;
  }
  float* op = static_cast<float*>(a.o) + static_cast<int64_t>(T) * a.s * a.b * a.nh * DH +
              (static_cast<int64_t>(q) * a.b + bi) * a.nh * DH + h * DH + j * H;
  // a row that sees no key: o = 0, lse = −∞
#pragma unroll
  for (int d = 0; d < H; ++d) op[d] = l > 0.f ? acc[d] / l : 0.f;
  if (j == 0)
    a.lse[((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s + q] = l > 0.f ? m + logf(l) : -INFINITY;
}

// ------------------------------------------------------------------ backward
struct AttnBwdArgs {
  const void* qkv;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;
  void* dqkv;
  int s, b, nh, T;
  int nqb;            // blocks of AQ rows (dq workgroups, dk/dv workgroups)
  float scale, scale_log2;
  uint32_t qkv_shard_bytes, o_shard_bytes;
  const uint32_t* mask;  // packed general mask (2 parts of [b][s][mw] words), or null
  int mw;                // words per position, ⌈s/32⌉
};

// δ[T][bi][h][q] = Σ_d do·o over the head's dh columns of row q (fp32): one
// thread per (shard, token row, head).
template <typename TT, int DH>
__global__ __launch_bounds__(256) void attn_delta_kernel(AttnBwdArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(a.s) * a.b;
  if (idx >= static_cast<int64_t>(a.T) * n * a.nh) return;
  const int h = static_cast<int>(idx % a.nh);
  const int64_t tr = idx / a.nh;  // T·n + token row
  const int T = static_cast<int>(tr / n);
  const int64_t r = tr % n;
  const int q = static_cast<int>(r / a.b), bi = static_cast<int>(r % a.b);
  const int64_t off = tr * a.nh * DH + static_cast<int64_t>(h) * DH;
  const TT* op = static_cast<const TT*>(a.o) + off;
  const TT* dp = static_cast<const TT*>(a.dout) + off;
  float acc = 0.f;
  if constexpr (sizeof(TT) == 2) {
#pragma unroll
    for (int c = 0; c < DH / 8; ++c) {
      const bf16x8 x = reinterpret_cast<const bf16x8*>(op)[c];
      const bf16x8 y = reinterpret_cast<const bf16x8*>(dp)[c];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(bf2f(x[e]), bf2f(y[e]), acc);
    }
  } else {
#pragma unroll
    for (int d = 0; d < DH; ++d) acc = fmaf(op[d], dp[d], acc);
  }
  a.delta[((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s + q] = acc;
}

// dq: a workgroup takes 128 query rows of one (shard, batch entry, head), a
// wave 32, with q, do and o fragments in registers; K and V tiles of 64 keys
// stream through LDS.  δ = rowsum(do ⊙ o) is formed here from the registers
// and written to the workspace for the dk/dv kernel, which runs after.  Per
// 32-key half of a tile: Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ (lane L holds query row
// L%32), P = exp2(S·log2(e)/√dh − lse·log2(e)), dS = P ⊙ (dP − δ), and
// dQᵀ += Kᵀ·dSᵀ with the keys in the accumulators' order.
template <int DH, bool CAUSAL, bool GMASK>
__global__ __launch_bounds__(ATHR, 2) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int TILE = AKV * DH * 2;
  constexpr int NC = DH / 16, ND = DH / 32;
  constexpr int NI = TILE / 1024 / 4;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  TPMLP_LDS char* lds = (TPMLP_LDS char*)(smem);
  int T, bi, h, p;
  attn_block<CAUSAL>(a.nh, a.b, a.nqb, T, bi, h, p);
  const int qb = a.nqb - 1 - p;  // the last query blocks see the most keys
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * AQ + wave * 32, qrow = q0 + r32;
  const int64_t row_len = static_cast<int64_t>(a.nh) * 3 * DH, orow = static_cast<int64_t>(a.nh) * DH;
  const int64_t n = static_cast<int64_t>(a.s) * a.b;
  const bf16* qkv = static_cast<const bf16*>(a.qkv) + T * n * row_len;
  const i32x4 rsrc = make_rsrc(qkv, a.qkv_shard_bytes);
  const int64_t kcol = static_cast<int64_t>(h) * 3 * DH + DH, vcol = kcol + DH;
  const int kv_end = CAUSAL ? min(a.s, qb * AQ + AQ) : a.s;
  const int nkv = (kv_end + AKV - 1) / AKV;

  load_tile<DH>(rsrc, lds, a.s, a.b, bi, row_len, kcol, 0, wave, lane);
  load_tile<DH>(rsrc, lds + TILE, a.s, a.b, bi, row_len, vcol, 0, wave, lane);

  bf16x8 qf[NC], df[NC];
  const bool valid = qrow < a.s;
  const int64_t srow = ((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s;
  float dlt = 0.f;
  if constexpr (!GMASK) {
    // The wave's 32 rows of q, dO and o, loaded as whole rows (16-B chunk
    // lane % CPR of row lane / CPR + RPI·i; rows past s read as zeros) and
    // passed through the wave's region of stage 1 (free until the first
    // step's barrier) into the fragment layout: lane (r32, hi) needs chunks
    // 2c + hi of row r32.  Each lane loading its own chunks would make every
    // load touch 32 rows.
    constexpr int RB = DH * 2, CPR = DH / 8, RPI = 64 / CPR, NS = 32 / RPI;
    const int rr = lane / CPR, ch = lane % CPR;
    const i32x4 rdo = make_rsrc(static_cast<const bf16*>(a.dout) + T * n * orow, a.o_shard_bytes);
    const i32x4 ro = make_rsrc(static_cast<const bf16*>(a.o) + T * n * orow, a.o_shard_bytes);
    i32x4 lq[NS], ld[NS], lo[NS];
    auto ooff = [&](int i) {
      const int R = q0 + rr + RPI * i;
      return R < a.s ? static_cast<int>(((static_cast<int64_t>(R) * a.b + bi) * orow + h * DH + 8 * ch) * 2)
                     : static_cast<int>(AOOB);
    };
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int R = q0 + rr + RPI * i;
      const int64_t tok = static_cast<int64_t>(R) * a.b + bi;
      lq[i] = tpmlp_llvm_buffer_load_v4(
          rsrc, R < a.s ? static_cast<int>((tok * row_len + h * 3 * DH + 8 * ch) * 2) : static_cast<int>(AOOB), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) ld[i] = tpmlp_llvm_buffer_load_v4(rdo, ooff(i), 0, 0);
    const uint32_t reg = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + 2 * TILE + wave * 32 * RB;
    auto to_frags = [&](const i32x4(&x)[NS], bf16x8(&out)[NC]) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        asm volatile("ds_write_b128 %0, %1" ::"v"(reg + kv_slot<DH>(rr + RPI * i, ch)), "v"(x[i]) : "memory");
      lds_wait();
      i32x4 f[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) f[c] = lds_rd128<0>(reg + kv_slot<DH>(r32, 2 * c + hi));
      lds_wait();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        asm volatile("" : "+v"(f[c]));
        out[c] = __builtin_bit_cast(bf16x8, f[c]);
      }
    };
    // o (needed only for δ) is loaded once q is staged, so that at most two
    // of the three row sets are live at a time
    bf16x8 of[NC];
    to_frags(lq, qf);
#pragma unroll
    for (int i = 0; i < NS; ++i) lo[i] = tpmlp_llvm_buffer_load_v4(ro, ooff(i), 0, 0);
    to_frags(ld, df);
    to_frags(lo, of);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = fmaf(bf2f(df[c][e]), bf2f(of[c][e]), dlt);
  } else {
    // (the general-mask kernel keeps per-lane fragment loads: the staged
    // form's registers made it spill)
    const int64_t tok = static_cast<int64_t>(qrow) * a.b + bi;
    const bf16* qp = qkv + tok * row_len + h * 3 * DH + 8 * hi;
    const int64_t oo = T * n * orow + tok * orow + h * DH + 8 * hi;
    const bf16* dp = static_cast<const bf16*>(a.dout) + oo;
    const bf16* op = static_cast<const bf16*>(a.o) + oo;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = valid ? *reinterpret_cast<const bf16x8*>(qp + 16 * c) : bf16x8{};
      df[c] = valid ? *reinterpret_cast<const bf16x8*>(dp + 16 * c) : bf16x8{};
      const bf16x8 of = valid ? *reinterpret_cast<const bf16x8*>(op + 16 * c) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = fmaf(bf2f(df[c][e]), bf2f(of[e]), dlt);
    }
  }
  dlt += __shfl_xor(dlt, 32, 64);
  if (valid && hi == 0) a.delta[srow + qrow] = dlt;
  // lse = −∞ (a row that sees no key, every entry hidden): +∞ here makes
  // P = 2^(−∞ − ∞) = 0 instead of NaN
  float lse2 = 0.f;
  if (valid) {
    const float l = a.lse[srow + qrow];
    lse2 = l == -INFINITY ? INFINITY : l * 1.4426950408889634f;
  }
  const i32x4 mrs = GMASK ? make_rsrc(a.mask + static_cast<int64_t>(bi) * a.s * a.mw,
                                        static_cast<uint32_t>(static_cast<int64_t>(a.s) * a.mw * 4))
                             : i32x4{0, 0, 0, 0};

  f32x16 dq[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[d][v] = 0.f;

  // row-fragment and transposed-read addresses (block offsets are immediates)
  constexpr int RB = DH * 2, NR = 2 * ND;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  uint32_t ro[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) ro[c] = lds_base + kv_slot<DH>(r32, 2 * c + hi);
  uint32_t va[NR];
  tr_addrs<DH, ND>(lds_base, lane, va);

  // general-mask words of key block jj for this lane's row (one per 32 keys)
  uint32_t mwn[2] = {~0u, ~0u};
  auto mask_words = [&](int jj) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pos = jj * AKV + 32 * u;
      mwn[u] = valid && pos < a.s ? tpmlp_llvm_buffer_load_u32(mrs, (qrow * a.mw + pos / 32) * 4, 0, 0) : ~0u;
    }
  };
  if constexpr (GMASK) mask_words(0);

  // One key block in stage ST (compile-time: every LDS offset is an
  // immediate).  One barrier per block: after it every wave has finished the
  // previous block, so the other stage is free and the next block's DMA is
  // issued into it, running during this block.
  auto step = [&](auto stc, int j) {
    constexpr int ST = decltype(stc)::value;
    wait_vmcnt<0>();  // this wave's share of block j
    lds_barrier();
    // a causal block whose first key is past the wave's last query row (or a
    // wave wholly past s) contributes nothing
    const int t0 = j * AKV;
    const bool dead = q0 >= a.s || (CAUSAL && t0 > q0 + 31);
    // general mask of the block's keys for this lane's row (bit v of mk[u]:
    // accumulator entry v of half u), from the words loaded one block ahead;
    // the next block's words are loaded before its DMA
    uint32_t mk[2] = {0u, 0u};
    bool hidden = false;
    if constexpr (GMASK) {
      mk[0] = lane_bits16(mwn[0], hi);
      mk[1] = lane_bits16(mwn[1], hi);
      if (j + 1 < nkv) mask_words(j + 1);
      hidden = __all((mk[0] & mk[1]) == 0xFFFFu);  // the wave sees no key of the block
    }
    if (j + 1 < nkv) {
      TPMLP_LDS char* nxt = lds + (ST ^ 1) * 2 * TILE;
      load_tile<DH>(rsrc, nxt, a.s, a.b, bi, row_len, kcol, j + 1, wave, lane);
      load_tile<DH>(rsrc, nxt + TILE, a.s, a.b, bi, row_len, vcol, j + 1, wave, lane);
    }
    if (dead || hidden) return;
    const bool masked = t0 + AKV > a.s || q0 + 31 >= a.s || (CAUSAL && t0 + AKV - 1 > q0);
    static_for<0, 2>([&](auto uc) {
      constexpr int U = decltype(uc)::value;
      constexpr int KB = ST * 2 * TILE + U * 32 * RB, VB = KB + TILE;  // key rows 32U.. of K and V
      // Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ for the lane's query row: slices read
      // three ahead
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] = pacc[v] = 0.f;
      i32x4 kr[4], vr[4];
      auto rd2 = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
        kr[c % 4] = lds_rd128<KB>(ro[c]);
        vr[c % 4] = lds_rd128<VB>(ro[c]);
      };
      static_for<0, (NC < 3 ? NC : 3)>(rd2);
      static_for<0, NC>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        constexpr int later = 2 * (NC - 1 - c < 2 ? NC - 1 - c : 2);
        lgkm_wait<later>(kr[c % 4], vr[c % 4]);
        sacc = mfma(__builtin_bit_cast(bf16x8, kr[c % 4]), qf[c], sacc);
        pacc = mfma(__builtin_bit_cast(bf16x8, vr[c % 4]), df[c], pacc);
        if constexpr (c + 3 < NC) rd2(ic<c + 3>{});
      });
      // both transposed K blocks are read while dS is formed
      i32x2 ta[NR], tb[NR];
      tr_issue<DH, ND, KB>(va, ta);
      tr_issue<DH, ND, KB + 16 * RB>(va, tb);
      if (masked) {
        const int lim = valid ? (CAUSAL ? min(qrow + 1, a.s) : a.s) : 0;
        mask_range1(sacc, U, -1 << 30, lim - t0 - 4 * hi, -INFINITY);
      }
      if constexpr (GMASK) apply_mask16(sacc, mk[U]);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], a.scale_log2, -lse2));
        sacc[v] = p * (pacc[v] - dlt);  // dS
      }
      bf16x8 kt[ND];
      tr_wait<NR, ND>(ta);
      tr_frags<ND>(ta, kt);
      {
        const bf16x8 sf = pack_acc(sacc, 0);
#pragma unroll
        for (int d = 0; d < ND; ++d) dq[d] = mfma(kt[d], sf, dq[d]);
      }
      tr_wait<0, ND>(tb);
      tr_frags<ND>(tb, kt);
      {
        const bf16x8 sf = pack_acc(sacc, 1);
#pragma unroll
        for (int d = 0; d < ND; ++d) dq[d] = mfma(kt[d], sf, dq[d]);
      }
    });
  };
  int j = 0;
  for (; j + 1 < nkv; j += 2) {
    step(ic<0>{}, j);
    step(ic<1>{}, j + 1);
  }
  if (j < nkv) step(ic<0>{}, j);
  // dq, staged through the stage the last block did not use (free since its
  // barrier), one 32-row region per wave
  bf16* op = static_cast<bf16*>(a.dqkv) + T * n * row_len + (static_cast<int64_t>(q0) * a.b + bi) * row_len +
             h * 3 * DH;
  store_rows_staged<DH>(dq, a.scale, lds_base + (nkv & 1) * 2 * TILE + wave * 32 * RB, op,
                        static_cast<int64_t>(a.b) * row_len, a.s - q0, lane);
}

// dk, dv: a workgroup takes 128 key rows, a wave 32, with k and v fragments in
// registers; Q and dO tiles of 64 query rows (and their lse, δ) stream
// through LDS.  Per 32-query half of a tile: S'ᵀ = Q·Kᵀ and dP'ᵀ = dO·Vᵀ
// with lane L holding key row L%32, P and dS as in dq, then dVᵀ += dOᵀ·P and
// dKᵀ += Qᵀ·dS with the query rows in the accumulators' order.
template <int DH, bool CAUSAL, bool GMASK>
__global__ __launch_bounds__(ATHR, DH == 128 ? 1 : 2) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int TILE = AKV * DH * 2;
  constexpr int NC = DH / 16, ND = DH / 32;
  constexpr int NI = TILE / 1024 / 4;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  __shared__ __attribute__((aligned(1024))) char kvmem[4 * TILE];  // the workgroup's 128 K rows, then V rows
  __shared__ __attribute__((aligned(16))) float stat[2][2][AKV];  // [stage][lse·log2(e) | δ][row]
  TPMLP_LDS char* lds = (TPMLP_LDS char*)(smem);
  int T, bi, h, kb_idx;
  attn_block<CAUSAL>(a.nh, a.b, a.nqb, T, bi, h, kb_idx);  // the first key blocks see the most query blocks
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi = lane >> 5;
  const int k0 = kb_idx * AQ + wave * 32, krow = k0 + r32;
  const int64_t row_len = static_cast<int64_t>(a.nh) * 3 * DH, orow = static_cast<int64_t>(a.nh) * DH;
  const int64_t n = static_cast<int64_t>(a.s) * a.b;
  const bf16* qkv = static_cast<const bf16*>(a.qkv) + T * n * row_len;
  const bf16* dout = static_cast<const bf16*>(a.dout) + T * n * orow;
  const i32x4 rq = make_rsrc(qkv, a.qkv_shard_bytes);
  const i32x4 rd = make_rsrc(dout, a.o_shard_bytes);
  const int64_t qcol = static_cast<int64_t>(h) * 3 * DH, dcol = static_cast<int64_t>(h) * DH;
  const int64_t srow = ((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s;
  const int j0 = CAUSAL ? (kb_idx * AQ) / AKV : 0;
  const int nq = (a.s + AKV - 1) / AKV;

  // statistics of query block j (threads 0..127: one value each)
  auto load_stat = [&](int j, float& v) {
    const int t = threadIdx.x & 63, qr = j * AKV + t;
    if (threadIdx.x < 64) {
      // lse = −∞ (a row that sees no key): +∞ makes its P = 0 instead of NaN
      const float l = qr < a.s ? a.lse[srow + qr] : 0.f;
      v = l == -INFINITY ? INFINITY : l * 1.4426950408889634f;
    }
    else if (threadIdx.x < 128) v = qr < a.s ? a.delta[srow + qr] : 0.f;
  };
  auto store_stat = [&](int st, float v) {
    if (threadIdx.x < 128) stat[st][threadIdx.x >> 6][threadIdx.x & 63] = v;
  };

  float sv = 0.f;
  load_stat(j0, sv);
  load_tile<DH>(rq, lds, a.s, a.b, bi, row_len, qcol, j0, wave, lane);
  load_tile<DH>(rd, lds + TILE, a.s, a.b, bi, orow, dcol, j0, wave, lane);
  // the workgroup's 128 keys: their K and V rows (two 64-row tiles each, rows
  // past s zero-filled) by DMA into their own region, whole rows per load;
  // each lane loading its own fragments would touch 32 rows per load, and
  // with one workgroup per CU nothing else runs while they arrive
  TPMLP_LDS char* kvl = (TPMLP_LDS char*)(kvmem);
  load_tile<DH>(rq, kvl, a.s, a.b, bi, row_len, qcol + DH, 2 * kb_idx, wave, lane);
  load_tile<DH>(rq, kvl + TILE, a.s, a.b, bi, row_len, qcol + DH, 2 * kb_idx + 1, wave, lane);
  load_tile<DH>(rq, kvl + 2 * TILE, a.s, a.b, bi, row_len, qcol + 2 * DH, 2 * kb_idx, wave, lane);
  load_tile<DH>(rq, kvl + 3 * TILE, a.s, a.b, bi, row_len, qcol + 2 * DH, 2 * kb_idx + 1, wave, lane);

  // k and v fragments of the lane's key, kept in AGPRs (an MFMA operand may
  // come from either register file; the VGPRs go to the S and dP
  // accumulators, which the VALU reads)
  i32x4 kf[NC], vf[NC];
  const bool valid = krow < a.s;
  // this batch entry's general mask (read only when GMASK and krow < s)
  const i32x4 mrs = GMASK ? make_rsrc(a.mask + (static_cast<int64_t>(a.b) + bi) * a.s * a.mw,
                                        static_cast<uint32_t>(static_cast<int64_t>(a.s) * a.mw * 4))
                             : i32x4{0, 0, 0, 0};
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[d][v] = dv[d][v] = 0.f;
  wait_vmcnt<0>();
  store_stat(0, sv);

  // row-fragment and transposed-read addresses (block offsets are immediates)
  constexpr int RB = DH * 2, NR = 2 * ND;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  uint32_t ro[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) ro[c] = lds_base + kv_slot<DH>(r32, 2 * c + hi);
  uint32_t va[NR];
  tr_addrs<DH, ND>(lds_base, lane, va);
  {
    // the wave's 32 keys are rows 32·(wave % 2) .. of K (V) tile wave / 2
    lds_barrier();  // every wave's share of the K and V rows has landed
    const uint32_t kvb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(kvl)) + (wave >> 1) * TILE +
                         (wave & 1) * 32 * RB;
    i32x4 kr[NC], vr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kr[c] = lds_rd128<0>(kvb + kv_slot<DH>(r32, 2 * c + hi));
      vr[c] = lds_rd128<2 * TILE>(kvb + kv_slot<DH>(r32, 2 * c + hi));
    }
    lds_wait();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      asm volatile("" : "+v"(kr[c]), "+v"(vr[c]));
      kf[c] = kr[c];
      vf[c] = vr[c];
      asm volatile("" : "+a"(kf[c]), "+a"(vf[c]));
    }
  }
  // this lane's statistics: 4 consecutive query rows per 16-B read
  const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&stat[0][0][0])) + 16 * hi;

  // general-mask words of query block jj for this lane's key (column part,
  // one per 32 query rows)
  uint32_t mwn[2] = {~0u, ~0u};
  auto mask_words = [&](int jj) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pos = jj * AKV + 32 * u;
      mwn[u] = valid && pos < a.s ? tpmlp_llvm_buffer_load_u32(mrs, (krow * a.mw + pos / 32) * 4, 0, 0) : ~0u;
    }
  };
  if constexpr (GMASK) mask_words(j0);

  // One query block in stage ST (compile-time: every LDS offset is an
  // immediate).  One barrier per block: after it every wave has finished the
  // previous block, so the other stage (tiles and statistics) is free; the
  // next block's DMA and statistics loads are issued into it and run during
  // this block.
  auto step = [&](auto stc, int j) {
    constexpr int ST = decltype(stc)::value;
    wait_vmcnt<0>();  // this wave's share of block j and its statistic
    lds_wait();       // its statistics write of the previous step
    lds_barrier();
    const int t0 = j * AKV;
    const bool masked = t0 + AKV > a.s || k0 + 31 >= a.s || (CAUSAL && t0 < k0 + 31);
    // a causal block whose last query row is before the wave's first key (or
    // a wave wholly past s) contributes nothing
    const bool dead = k0 >= a.s || (CAUSAL && t0 + AKV - 1 < k0);
    // general mask of (query row, this lane's key), from the packed mask's
    // column part: bit v of mk[U] for accumulator entry v, query row t0 + 32U +
    // 8(v/4) + 4·hi + v%4; from the words loaded one block ahead, the next
    // block's words loaded before its DMA
    uint32_t mk[2] = {0u, 0u};
    bool hidden = false;
    if constexpr (GMASK) {
      mk[0] = lane_bits16(mwn[0], hi);
      mk[1] = lane_bits16(mwn[1], hi);
      if (j + 1 < nq) mask_words(j + 1);
      hidden = __all((mk[0] & mk[1]) == 0xFFFFu);  // no query of the block sees the wave's keys
    }
    if (j + 1 < nq) {
      load_stat(j + 1, sv);
      TPMLP_LDS char* nxt = lds + (ST ^ 1) * 2 * TILE;
      load_tile<DH>(rq, nxt, a.s, a.b, bi, row_len, qcol, j + 1, wave, lane);
      load_tile<DH>(rd, nxt + TILE, a.s, a.b, bi, orow, dcol, j + 1, wave, lane);
    }
    if (!dead && !hidden) static_for<0, 2>([&](auto uc) {
      constexpr int U = decltype(uc)::value;
      constexpr int QB = ST * 2 * TILE + U * 32 * RB, DB = QB + TILE;  // rows 32U.. of Q and dO
      // statistics of the lane's 16 query rows (lse·log2(e), δ), read ahead
      f32x4 ls[4], ds[4];
      i32x4 sr[8];
      static_for<0, 4>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        sr[g] = lds_rd128<((2 * ST + 0) * AKV + 32 * U + 8 * g) * 4>(sbase);
        sr[4 + g] = lds_rd128<((2 * ST + 1) * AKV + 32 * U + 8 * g) * 4>(sbase);
      });
      // S = Q·Kᵀ and dP = dO·Vᵀ for the lane's key: slices read three ahead.
      // The products are inline asm with VGPR accumulators (the compiler's
      // form for this one-wave-per-SIMD kernel keeps them in AGPRs, and every
      // VALU use below would first copy them out); the first slice starts
      // from zero.
      f32x16 sacc, pacc;
      i32x4 qr[4], dr[4];
      auto rd2 = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
        qr[c % 4] = lds_rd128<QB>(ro[c]);
        dr[c % 4] = lds_rd128<DB>(ro[c]);
      };
      static_for<0, (NC < 3 ? NC : 3)>(rd2);
      static_for<0, NC>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        constexpr int later = 2 * (NC - 1 - c < 2 ? NC - 1 - c : 2);
        lgkm_wait<later>(qr[c % 4], dr[c % 4]);
        if constexpr (c == 0) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(qr[0]), "a"(kf[0]));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(pacc) : "v"(dr[0]), "a"(vf[0]));
        } else {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(qr[c % 4]), "a"(kf[c]));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(pacc) : "v"(dr[c % 4]), "a"(vf[c]));
        }
        if constexpr (c + 3 < NC) rd2(ic<c + 3>{});
      });
      // the VALU reads the results only after the MFMA pipeline has written
      // them (the wait states the compiler inserts for its own MFMAs)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(sacc), "+v"(pacc));
      // every LDS read above is complete (the last wait was for zero)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        asm volatile("" : "+v"(sr[g]), "+v"(sr[4 + g]));
        ls[g] = __builtin_bit_cast(f32x4, sr[g]);
        ds[g] = __builtin_bit_cast(f32x4, sr[4 + g]);
      }
      // the first two transposed blocks are read while P and dS are formed
      i32x2 ta[NR], tb[NR];
      tr_issue<DH, ND, DB>(va, ta);
      tr_issue<DH, ND, QB>(va, tb);
      // lane: key krow, query rows 64j + 32U + 8(v/4) + 4·hi + v%4; the
      // mask runs only on tiles that reach past s, past this wave's keys'
      // diagonal, or hold key rows past s
      if (masked) {
        const int lo = CAUSAL ? krow - t0 - 4 * hi : -1 << 30;
        const int hi_ = valid ? a.s - t0 - 4 * hi : lo;
        mask_range1(sacc, U, lo, hi_, -INFINITY);
      }
      if constexpr (GMASK) apply_mask16(sacc, mk[U]);
      f32x16 pv;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g + e;
          pv[v] = __builtin_amdgcn_exp2f(fmaf(sacc[v], a.scale_log2, -ls[g][e]));
          sacc[v] = pv[v] * (pacc[v] - ds[g][e]);  // dS
        }
      // dv += Pᵀ·dO and dk += dSᵀ·Q over the block's 32 query rows, 16 at a
      // time; block g + 1's reads are in flight during block g's MFMAs
      bf16x8 ft[ND];
      tr_wait<NR, ND>(ta);
      tr_frags<ND>(ta, ft);
      {
        const bf16x8 pf = pack_acc(pv, 0);
#pragma unroll
        for (int d = 0; d < ND; ++d) dv[d] = mfma(ft[d], pf, dv[d]);
      }
      tr_issue<DH, ND, DB + 16 * RB>(va, ta);
      tr_wait<NR, ND>(tb);
      tr_frags<ND>(tb, ft);
      {
        const bf16x8 sf = pack_acc(sacc, 0);
#pragma unroll
        for (int d = 0; d < ND; ++d) dk[d] = mfma(ft[d], sf, dk[d]);
      }
      tr_issue<DH, ND, QB + 16 * RB>(va, tb);
      tr_wait<NR, ND>(ta);
      tr_frags<ND>(ta, ft);
      {
        const bf16x8 pf = pack_acc(pv, 1);
#pragma unroll
        for (int d = 0; d < ND; ++d) dv[d] = mfma(ft[d], pf, dv[d]);
      }
      tr_wait<0, ND>(tb);
      tr_frags<ND>(tb, ft);
      {
        const bf16x8 sf = pack_acc(sacc, 1);
#pragma unroll
        for (int d = 0; d < ND; ++d) dk[d] = mfma(ft[d], sf, dk[d]);
      }
    });
    // the next block's statistics go into the other stage (read after the
    // next barrier)
    if (j + 1 < nq) store_stat(ST ^ 1, sv);
  };
  int j = j0;
  for (; j + 1 < nq; j += 2) {
    step(ic<0>{}, j);
    step(ic<1>{}, j + 1);
  }
  if (j < nq) step(ic<0>{}, j);
  // dk then dv, each staged through the wave's region of the stage the last
  // block did not use (free since its barrier; the statistics have their own
  // array), the second after the first one's reads have completed
  bf16* op = static_cast<bf16*>(a.dqkv) + T * n * row_len + (static_cast<int64_t>(k0) * a.b + bi) * row_len +
             h * 3 * DH + DH;
  const uint32_t reg = lds_base + ((nq - j0) & 1) * 2 * TILE + wave * 32 * RB;
  store_rows_staged<DH>(dk, a.scale, reg, op, static_cast<int64_t>(a.b) * row_len, a.s - k0, lane);
  store_rows_staged<DH>(dv, 1.0f, reg, op + DH, static_cast<int64_t>(a.b) * row_len, a.s - k0, lane);
}


__device__ void tpmlp_llvm_buffer_store_v4(i32x4 vdata, i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.store.v4i32");

// store_rows_staged with buffer stores: exactly 32·DH/512 store instructions
// per call whatever nrows is (rows past it go past the buffer's range)
template <int DH>
__device__ __forceinline__ void store_rows_staged_buf(const f32x16 (&acc)[DH / 32], float scale, uint32_t reg,
                                                      i32x4 rs, int64_t off0, int64_t ldb, int nrows, int lane) {
  constexpr int RB = DH * 2, GS = DH == 128 ? 0 : 1;
  constexpr int CPR = DH / 8, RPI = 64 / CPR, NS = 32 / RPI;
  const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int d = 0; d < DH / 32; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = f2bf(acc[d][4 * q4 + e] * scale);
      const uint32_t ad = reg + r32 * RB + (((2 * (4 * d + q4) + hi) ^ (r32 >> GS)) << 3);
      asm volatile("ds_write_b64 %0, %1" ::"v"(ad), "v"(__builtin_bit_cast(i32x2, w)) : "memory");
    }
  lds_wait();
  const int mc = lane % CPR;
  i32x4 v[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int R = i * RPI + lane / CPR;
    v[i] = lds_rd128<0>(reg + R * RB + (((2 * mc) ^ (R >> GS)) & ~1) * 8);
  }
  lds_wait();
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    asm volatile("" : "+v"(v[i]));
    const int R = i * RPI + lane / CPR;
    if ((R >> GS) & 1) v[i] = i32x4{v[i][2], v[i][3], v[i][0], v[i][1]};
    tpmlp_llvm_buffer_store_v4(v[i], rs, R < nrows ? static_cast<int>(off0 + R * ldb + 16 * mc) : static_cast<int>(AOOB),
                               0, 0);
  }
}

// dk/dv, persistent: gridDim.x = 8·W workgroups, workgroup (x = wg % 8,
// l = wg / 8) takes the key blocks of XCD x at local positions l, 2W-1-l,
// 2W+l, ... of the longest-first list (G blocks in all).  While a block runs,
// the next block's K and V rows (from its first step) and its first query
// tile and statistics (in its last step) are loaded, so the next block starts
// without waiting for memory, and this block's stores stay in flight while it
// starts: its first wait lets exactly the 2·NS stores be outstanding (loads
// and stores leave the vector-memory counter in issue order).
constexpr unsigned kDkdvPersistWG = 256;  // one workgroup per CU (8 XCDs × 32)

template <int DH, bool CAUSAL>
__global__ __launch_bounds__(ATHR, DH == 128 ? 1 : 2) void attn_bwd_dkdv_pkernel(AttnBwdArgs a, int G) {
  static_assert(DH == 128, "the persistent dk/dv kernel is built for dh 128 (one workgroup per CU)");
  constexpr int TILE = AKV * DH * 2;
  constexpr int NC = DH / 16, ND = DH / 32;
  constexpr int RB = DH * 2, NR = 2 * ND;
  constexpr int NS = 32 / (64 / (DH / 8));
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  __shared__ __attribute__((aligned(1024))) char kvmem[4 * TILE];
  __shared__ __attribute__((aligned(16))) float stat[2][2][AKV];
  TPMLP_LDS char* lds = (TPMLP_LDS char*)(smem);
  TPMLP_LDS char* kvl = (TPMLP_LDS char*)(kvmem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi = lane >> 5;
  const int64_t row_len = static_cast<int64_t>(a.nh) * 3 * DH, orow = static_cast<int64_t>(a.nh) * DH;
  const int64_t n = static_cast<int64_t>(a.s) * a.b;
  const int nq = (a.s + AKV - 1) / AKV;
  const int W = static_cast<int>(gridDim.x) >> 3;
  const int xcd = static_cast<int>(blockIdx.x) & 7, l = static_cast<int>(blockIdx.x) >> 3;
  auto vblock = [&](int r) {
    const int loc = (r & 1) ? (r + 1) * W - 1 - l : r * W + l;
    return loc * 8 + xcd;
  };
  // a block: shard, batch entry, head, key block (everything else follows)
  struct Blk {
    int T, bi, h, kb;
    __device__ int j0() const { return CAUSAL ? (kb * AQ) / AKV : 0; }
    __device__ int64_t srow(const AttnBwdArgs& a) const {
      return ((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s;
    }
  };
  auto make_blk = [&](int vb) {
    Blk B;
    attn_block_at<CAUSAL>(a.nh, a.b, a.nqb, G, vb, B.T, B.bi, B.h, B.kb);
    return B;
  };
  auto rs_qkv = [&](const Blk& B) {
    return make_rsrc(static_cast<const bf16*>(a.qkv) + B.T * n * row_len, a.qkv_shard_bytes);
  };
  auto rs_dout = [&](const Blk& B) {
    return make_rsrc(static_cast<const bf16*>(a.dout) + B.T * n * orow, a.o_shard_bytes);
  };
  auto load_stat = [&](const Blk& B, int j, float& v) {
    const int t = threadIdx.x & 63, qr = j * AKV + t;
    const int64_t sr = B.srow(a);
    if (threadIdx.x < 64) {
      const float lv = qr < a.s ? a.lse[sr + qr] : 0.f;
      v = lv == -INFINITY ? INFINITY : lv * 1.4426950408889634f;
    } else if (threadIdx.x < 128) v = qr < a.s ? a.delta[sr + qr] : 0.f;
  };
  auto store_stat = [&](int st, float v) {
    if (threadIdx.x < 128) stat[st][threadIdx.x >> 6][threadIdx.x & 63] = v;
  };
  auto load_kv = [&](const Blk& B) {
    const i32x4 rq = rs_qkv(B);
    const int64_t kc = static_cast<int64_t>(B.h) * 3 * DH + DH;
    load_tile<DH>(rq, kvl, a.s, a.b, B.bi, row_len, kc, 2 * B.kb, wave, lane);
    load_tile<DH>(rq, kvl + TILE, a.s, a.b, B.bi, row_len, kc, 2 * B.kb + 1, wave, lane);
    load_tile<DH>(rq, kvl + 2 * TILE, a.s, a.b, B.bi, row_len, kc + DH, 2 * B.kb, wave, lane);
    load_tile<DH>(rq, kvl + 3 * TILE, a.s, a.b, B.bi, row_len, kc + DH, 2 * B.kb + 1, wave, lane);
  };
  auto load_q = [&](const Blk& B, int j, TPMLP_LDS char* dst) {
    load_tile<DH>(rs_qkv(B), dst, a.s, a.b, B.bi, row_len, static_cast<int64_t>(B.h) * 3 * DH, j, wave, lane);
    load_tile<DH>(rs_dout(B), dst + TILE, a.s, a.b, B.bi, orow, static_cast<int64_t>(B.h) * DH, j, wave, lane);
  };
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  uint32_t ro[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) ro[c] = lds_base + kv_slot<DH>(r32, 2 * c + hi);
  uint32_t va[NR];
  tr_addrs<DH, ND>(lds_base, lane, va);
  const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&stat[0][0][0])) + 16 * hi;
  const uint32_t kvb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(kvl)) + (wave >> 1) * TILE +
                       (wave & 1) * 32 * RB;

  Blk cur = make_blk(vblock(0));
  bool has_next = vblock(1) < G;
  Blk nxt = has_next ? make_blk(vblock(1)) : cur;
  float sv = 0.f;
  load_stat(cur, cur.j0(), sv);
  load_q(cur, cur.j0(), lds);
  load_kv(cur);
  wait_vmcnt<0>();
  store_stat(0, sv);
  int st0 = 0;
  i32x4 kf[NC], vf[NC];
  f32x16 dk[ND], dv[ND];
  for (int r = 0;; ++r) {
    // this block's k and v fragments from the K/V rows in kvmem
    lds_barrier();
    {
      i32x4 kr[NC], vr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        kr[c] = lds_rd128<0>(kvb + kv_slot<DH>(r32, 2 * c + hi));
        vr[c] = lds_rd128<2 * TILE>(kvb + kv_slot<DH>(r32, 2 * c + hi));
      }
      lds_wait();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        asm volatile("" : "+v"(kr[c]), "+v"(vr[c]));
        kf[c] = kr[c];
        vf[c] = vr[c];
        asm volatile("" : "+a"(kf[c]), "+a"(vf[c]));
      }
    }
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) dk[d][v] = dv[d][v] = 0.f;
    const int k0 = cur.kb * AQ + wave * 32, krow = k0 + r32, j0 = cur.j0();
    const bool valid = krow < a.s;

    auto step = [&](auto stc, int j, bool cont) {
      constexpr int ST = decltype(stc)::value;
      if (!cont) wait_vmcnt<0>();  // this wave's share of block j and its statistic
      lds_wait();
      lds_barrier();
      const int t0 = j * AKV;
      const bool masked = t0 + AKV > a.s || k0 + 31 >= a.s || (CAUSAL && t0 < k0 + 31);
      const bool dead = k0 >= a.s || (CAUSAL && t0 + AKV - 1 < k0);
      if (j + 1 < nq) {
        load_stat(cur, j + 1, sv);
        load_q(cur, j + 1, lds + (ST ^ 1) * 2 * TILE);
      } else if (has_next) {
        load_stat(nxt, nxt.j0(), sv);
        load_q(nxt, nxt.j0(), lds + (ST ^ 1) * 2 * TILE);
      }
      // kvmem is free once every wave has its fragments (before this barrier)
      if (j == j0 && has_next) load_kv(nxt);
    if (!dead) static_for<0, 2>([&](auto uc) {
      constexpr int U = decltype(uc)::value;
      constexpr int QB = ST * 2 * TILE + U * 32 * RB, DB = QB + TILE;  // rows 32U.. of Q and dO
      // statistics of the lane's 16 query rows (lse·log2(e), δ), read ahead
      f32x4 ls[4], ds[4];
      i32x4 sr[8];
      static_for<0, 4>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        sr[g] = lds_rd128<((2 * ST + 0) * AKV + 32 * U + 8 * g) * 4>(sbase);
        sr[4 + g] = lds_rd128<((2 * ST + 1) * AKV + 32 * U + 8 * g) * 4>(sbase);
      });
      // S = Q·Kᵀ and dP = dO·Vᵀ for the lane's key: slices read three ahead.
      // The products are inline asm with VGPR accumulators (the compiler's
      // form for this one-wave-per-SIMD kernel keeps them in AGPRs, and every
      // VALU use below would first copy them out); the first slice starts
      // from zero.
      f32x16 sacc, pacc;
      i32x4 qr[4], dr[4];
      auto rd2 = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
        qr[c % 4] = lds_rd128<QB>(ro[c]);
        dr[c % 4] = lds_rd128<DB>(ro[c]);
      };
      static_for<0, (NC < 3 ? NC : 3)>(rd2);
      static_for<0, NC>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        constexpr int later = 2 * (NC - 1 - c < 2 ? NC - 1 - c : 2);
        lgkm_wait<later>(qr[c % 4], dr[c % 4]);
        if constexpr (c == 0) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(qr[0]), "a"(kf[0]));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(pacc) : "v"(dr[0]), "a"(vf[0]));
        } else {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(qr[c % 4]), "a"(kf[c]));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(pacc) : "v"(dr[c % 4]), "a"(vf[c]));
        }
        if constexpr (c + 3 < NC) rd2(ic<c + 3>{});
      });
      // the VALU reads the results only after the MFMA pipeline has written
      // them (the wait states the compiler inserts for its own MFMAs)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(sacc), "+v"(pacc));
      // every LDS read above is complete (the last wait was for zero)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        asm volatile("" : "+v"(sr[g]), "+v"(sr[4 + g]));
        ls[g] = __builtin_bit_cast(f32x4, sr[g]);
        ds[g] = __builtin_bit_cast(f32x4, sr[4 + g]);
      }
      // the first two transposed blocks are read while P and dS are formed
      i32x2 ta[NR], tb[NR];
      tr_issue<DH, ND, DB>(va, ta);
      tr_issue<DH, ND, QB>(va, tb);
      // lane: key krow, query rows 64j + 32U + 8(v/4) + 4·hi + v%4; the
      // mask runs only on tiles that reach past s, past this wave's keys'
      // diagonal, or hold key rows past s
      if (masked) {
        const int lo = CAUSAL ? krow - t0 - 4 * hi : -1 << 30;
        const int hi_ = valid ? a.s - t0 - 4 * hi : lo;
        mask_range1(sacc, U, lo, hi_, -INFINITY);
      }
      f32x16 pv;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g + e;
          pv[v] = __builtin_amdgcn_exp2f(fmaf(sacc[v], a.scale_log2, -ls[g][e]));
          sacc[v] = pv[v] * (pacc[v] - ds[g][e]);  // dS
        }
      // dv += Pᵀ·dO and dk += dSᵀ·Q over the block's 32 query rows, 16 at a
      // time; block g + 1's reads are in flight during block g's MFMAs
      bf16x8 ft[ND];
      tr_wait<NR, ND>(ta);
      tr_frags<ND>(ta, ft);
      {
        const bf16x8 pf = pack_acc(pv, 0);
#pragma unroll
        for (int d = 0; d < ND; ++d) dv[d] = mfma(ft[d], pf, dv[d]);
      }
      tr_issue<DH, ND, DB + 16 * RB>(va, ta);
      tr_wait<NR, ND>(tb);
      tr_frags<ND>(tb, ft);
      {
        const bf16x8 sf = pack_acc(sacc, 0);
#pragma unroll
        for (int d = 0; d < ND; ++d) dk[d] = mfma(ft[d], sf, dk[d]);
      }
      tr_issue<DH, ND, QB + 16 * RB>(va, tb);
      tr_wait<NR, ND>(ta);
      tr_frags<ND>(ta, ft);
      {
        const bf16x8 pf = pack_acc(pv, 1);
#pragma unroll
        for (int d = 0; d < ND; ++d) dv[d] = mfma(ft[d], pf, dv[d]);
      }
      tr_wait<0, ND>(tb);
      tr_frags<ND>(tb, ft);
      {
        const bf16x8 sf = pack_acc(sacc, 1);
#pragma unroll
        for (int d = 0; d < ND; ++d) dk[d] = mfma(ft[d], sf, dk[d]);
      }
    });
      if (j + 1 < nq || has_next) store_stat(ST ^ 1, sv);
    };
    int j = j0;
    bool cont = r > 0;
    if (st0 == 0) {
      for (; j + 1 < nq; j += 2) {
        step(ic<0>{}, j, cont);
        cont = false;
        step(ic<1>{}, j + 1, false);
      }
      if (j < nq) step(ic<0>{}, j, cont);
    } else {
      for (; j + 1 < nq; j += 2) {
        step(ic<1>{}, j, cont);
        cont = false;
        step(ic<0>{}, j + 1, false);
      }
      if (j < nq) step(ic<1>{}, j, cont);
    }
    const int stl = (st0 + (nq - j0) - 1) & 1;  // the last step's stage
    lds_barrier();                                // every wave is done reading it
    const uint32_t reg = lds_base + stl * 2 * TILE + wave * 32 * RB;
    const i32x4 rw = make_rsrc(static_cast<bf16*>(a.dqkv) + cur.T * n * row_len, a.qkv_shard_bytes);
    const int64_t off0 = ((static_cast<int64_t>(k0) * a.b + cur.bi) * row_len + cur.h * 3 * DH + DH) * 2;
    store_rows_staged_buf<DH>(dk, a.scale, reg, rw, off0, static_cast<int64_t>(a.b) * row_len * 2, a.s - k0, lane);
    store_rows_staged_buf<DH>(dv, 1.0f, reg, rw, off0 + DH * 2, static_cast<int64_t>(a.b) * row_len * 2, a.s - k0,
                              lane);
    if (!has_next) break;
    // the next block's K/V rows, first query tile and statistics were issued
    // before the 2·NS stores above
    wait_vmcnt<2 * NS>();
    cur = nxt;
    st0 = stl ^ 1;
    has_next = vblock(r + 2) < G;
    if (has_next) nxt = make_blk(vblock(r + 2));
  }
}

// fp32 backward: dq per query row, dk and dv per key row, two lanes per row
// as in the forward (lane half j holds columns j·dh/2 ..).
template <int DH, bool CAUSAL>
__global__ __launch_bounds__(128) void attn_bwd_dq_f32_kernel(AttnBwdArgs a) {
  constexpr int H = DH / 2;
  const int64_t idx = (static_cast<int64_t>(blockIdx.x) * 128 + threadIdx.x) >> 1;
  const int j = threadIdx.x & 1;
  if (idx >= static_cast<int64_t>(a.T) * a.b * a.nh * a.s) return;  // both lanes of a pair
  const int q = static_cast<int>(idx % a.s);
  int64_t r = idx / a.s;
  const int h = static_cast<int>(r % a.nh);
  r /= a.nh;
  const int bi = static_cast<int>(r % a.b), T = static_cast<int>(r / a.b);
  const int64_t n = static_cast<int64_t>(a.s) * a.b;
  const int64_t row_len = static_cast<int64_t>(a.nh) * 3 * DH, orow = static_cast<int64_t>(a.nh) * DH;
  const float* qkv = static_cast<const float*>(a.qkv) + T * n * row_len;
  const float* qp = qkv + (static_cast<int64_t>(q) * a.b + bi) * row_len + h * 3 * DH + j * H;
  const float* dp = static_cast<const float*>(a.dout) + T * n * orow + (static_cast<int64_t>(q) * a.b + bi) * orow +
                    h * DH + j * H;
  const int64_t srow = ((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s;
  const float lse = a.lse[srow + q], dlt = a.delta[srow + q];
  float qv[H], dov[H], acc[H];
#pragma unroll
  for (int d = 0; d < H; ++d) {
    qv[d] = qp[d];
    dov[d] = dp[d];
    acc[d] = 0.f;
  }
  const int kend = CAUSAL ? q + 1 : a.s;
  const uint32_t* mrow = a.mask ? a.mask + (static_cast<int64_t>(bi) * a.s + q) * a.mw : nullptr;
  for (int kv = 0; kv < kend; ++kv) {
    if (mrow && ((mrow[kv >> 5] >> (kv & 31)) & 1u)) continue;  // hidden (all of them when lse = −∞)
    const float* kp = qkv + (static_cast<int64_t>(kv) * a.b + bi) * row_len + h * 3 * DH + DH + j * H;
    float sdot = 0.f, pdot = 0.f;
#pragma unroll
    for (int d = 0; d < H; ++d) {
      sdot = fmaf(qv[d], kp[d], sdot);
      pdot = fmaf(dov[d], kp[DH + d], pdot);
    }
    const float p = expf(pair_dot_sum<DH>(sdot) * a.scale - lse);
    const float ds = p * (pair_dot_sum<DH>(pdot) - dlt);
#pragma unroll
    for (int d = 0; d < H; ++d) acc[d] = fmaf(ds, kp[d], acc[d]);
  }
  float* op = static_cast<float*>(a.dqkv) + T * n * row_len + (static_cast<int64_t>(q) * a.b + bi) * row_len +
              h * 3 * DH + j * H;
#pragma unroll
  for (int d = 0; d < H; ++d) op[d] = acc[d] * a.scale;
}

template <int DH, bool CAUSAL>
__global__ __launch_bounds__(128) void attn_bwd_dkdv_f32_kernel(AttnBwdArgs a) {
  constexpr int H = DH / 2;
  const int64_t idx = (static_cast<int64_t>(blockIdx.x) * 128 + threadIdx.x) >> 1;
  const int j = threadIdx.x & 1;
  if (idx >= static_cast<int64_t>(a.T) * a.b * a.nh * a.s) return;  // both lanes of a pair
  const int kv = static_cast<int>(idx % a.s);
  int64_t r = idx / a.s;
  const int h = static_cast<int>(r % a.nh);
  r /= a.nh;
  const int bi = static_cast<int>(r % a.b), T = static_cast<int>(r / a.b);
  const int64_t n = static_cast<int64_t>(a.s) * a.b;
  const int64_t row_len = static_cast<int64_t>(a.nh) * 3 * DH, orow = static_cast<int64_t>(a.nh) * DH;
  const float* qkv = static_cast<const float*>(a.qkv) + T * n * row_len;
  const float* dout = static_cast<const float*>(a.dout) + T * n * orow;
  const float* kp = qkv + (static_cast<int64_t>(kv) * a.b + bi) * row_len + h * 3 * DH + DH + j * H;
  const int64_t srow = ((static_cast<int64_t>(T) * a.b + bi) * a.nh + h) * a.s;
  float kr[H], vr[H], dk[H], dv[H];
#pragma unroll
  for (int d = 0; d < H; ++d) {
    kr[d] = kp[d];
    vr[d] = kp[DH + d];
    dk[d] = dv[d] = 0.f;
  }
  const uint32_t* mcol = a.mask ? a.mask + ((static_cast<int64_t>(a.b) + bi) * a.s + kv) * a.mw : nullptr;
  for (int q = CAUSAL ? kv : 0; q < a.s; ++q) {
    if (mcol && ((mcol[q >> 5] >> (q & 31)) & 1u)) continue;  // the same for both lanes
    const float* qp = qkv + (static_cast<int64_t>(q) * a.b + bi) * row_len + h * 3 * DH + j * H;
    const float* dp = dout + (static_cast<int64_t>(q) * a.b + bi) * orow + h * DH + j * H;
    float sdot = 0.f, pdot = 0.f;
#pragma unroll
    for (int d = 0; d < H; ++d) {
      sdot = fmaf(qp[d], kr[d], sdot);
      pdot = fmaf(dp[d], vr[d], pdot);
    }
    const float p = expf(pair_dot_sum<DH>(sdot) * a.scale - a.lse[srow + q]);
    const float ds = p * (pair_dot_sum<DH>(pdot) - a.delta[srow + q]);
#pragma unroll
    for (int d = 0; d < H; ++d) {
      dv[d] = fmaf(p, dp[d], dv[d]);
      dk[d] = fmaf(ds, qp[d], dk[d]);
    }
  }
  float* op = static_cast<float*>(a.dqkv) + T * n * row_len + (static_cast<int64_t>(kv) * a.b + bi) * row_len +
              h * 3 * DH + DH + j * H;
#pragma unroll
  for (int d = 0; d < H; ++d) {
    op[d] = dk[d] * a.scale;
    op[DH + d] = dv[d];
  }
}

template <int DH, bool CAUSAL>
hipError_t launch_bwd_t(const AttnBwdArgs& a, int dt, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(a.T) * a.b * a.nh * a.s;
  hipError_t e;
  if (dt == 1) {
    // dq also forms δ (into the workspace) for the dk/dv kernel after it
    const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.T) * a.b * a.nh * a.nqb);
    if (a.mask) {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DH, CAUSAL, true>), dim3(blocks), dim3(ATHR), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DH, CAUSAL, true>), dim3(blocks), dim3(ATHR), 0, stream, a);
    } else {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DH, CAUSAL, false>), dim3(blocks), dim3(ATHR), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      // dh 128 (one workgroup per CU): the persistent kernel, one workgroup
      // per CU walking at least two key blocks; the block count is a multiple
      // of the 8 XCDs so that each XCD's share is its own list
      if (DH == 128 && blocks % 8 == 0 && blocks >= 2u * kDkdvPersistWG)
        hipLaunchKernelGGL((attn_bwd_dkdv_pkernel<128, CAUSAL>), dim3(kDkdvPersistWG), dim3(ATHR), 0, stream, a,
                           static_cast<int>(blocks));
      else
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DH, CAUSAL, false>), dim3(blocks), dim3(ATHR), 0, stream, a);
    }
  } else {
    const unsigned dblocks = static_cast<unsigned>((rows + 255) / 256);
    hipLaunchKernelGGL((attn_delta_kernel<float, DH>), dim3(dblocks), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned blocks = static_cast<unsigned>((2 * rows + 127) / 128);  // two lanes per row
    hipLaunchKernelGGL((attn_bwd_dkdv_f32_kernel<DH, CAUSAL>), dim3(blocks), dim3(128), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dq_f32_kernel<DH, CAUSAL>), dim3(blocks), dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

template <int DH, bool CAUSAL>
hipError_t launch_fwd_t(const AttnArgs& a, int dt, hipStream_t stream) {
  if (dt == 1) {
    const int64_t blocks = static_cast<int64_t>(a.T) * a.b * a.nh * a.nqb;
    if (a.mask)
      hipLaunchKernelGGL((attn_fwd_kernel<DH, CAUSAL, true>), dim3(static_cast<unsigned>(blocks)), dim3(ATHR), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<DH, CAUSAL, false>), dim3(static_cast<unsigned>(blocks)), dim3(ATHR), 0,
                         stream, a);
  } else {
    const int64_t total = static_cast<int64_t>(a.T) * a.b * a.nh * a.s;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<DH, CAUSAL>), dim3(static_cast<unsigned>((2 * total + 127) / 128)),
                       dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

// Bit-packing of a byte mask [b][s][s] (nonzero hides key j from query i):
// one thread per output word; part 0 (rows) reads 32 consecutive bytes of a
// row, part 1 (columns) 32 bytes of a column (adjacent threads take adjacent
// columns, so each of those reads is coalesced).  Positions past s are set.
__global__ __launch_bounds__(256) void attn_pack_mask_kernel(const uint8_t* __restrict__ mask,
                                                             uint32_t* __restrict__ out, int b, int s, int mw) {
  const int64_t per_part = static_cast<int64_t>(b) * s * mw;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= 2 * per_part) return;
  const int part = static_cast<int>(idx / per_part);
  int64_t r = idx - part * per_part;
  const int w = static_cast<int>(r % mw);
  r /= mw;
  const int pos = static_cast<int>(r % s), bi = static_cast<int>(r / s);
  const uint8_t* m = mask + static_cast<int64_t>(bi) * s * s;
  uint32_t word = 0;
  for (int j = 0; j < 32; ++j) {
    const int x = 32 * w + j;
    bool hid = true;
    if (x < s) hid = (part == 0 ? m[static_cast<int64_t>(pos) * s + x] : m[static_cast<int64_t>(x) * s + pos]) != 0;
    word |= static_cast<uint32_t>(hid) << j;
  }
  out[idx] = word;
}

}  // namespace

hipError_t launch_attn_pack_mask(int b, int s, const uint8_t* mask, uint32_t* packed, hipStream_t stream) {
  const int mw = (s + 31) / 32;
  const int64_t words = 2 * static_cast<int64_t>(b) * s * mw;
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_pack_mask_kernel, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, stream,
                     mask, packed, b, s, mw);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnProblem& p, hipStream_t stream) {
  AttnArgs a{};
  a.qkv = p.qkv;
  a.o = p.o;
  a.lse = p.lse;
  a.s = p.s;
  a.b = p.b;
  a.nh = p.nh;
  a.T = p.T;
  a.nqb = (p.s + AQ - 1) / AQ;
  a.scale = 1.0f / sqrtf(static_cast<float>(p.dh));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.qkv_shard_bytes = static_cast<uint32_t>(static_cast<int64_t>(p.s) * p.b * p.nh * 3 * p.dh * 2);
  a.mask = p.mask;
  a.mw = (p.s + 31) / 32;
  if (p.dh == 128)
    return p.causal ? launch_fwd_t<128, true>(a, p.dt, stream) : launch_fwd_t<128, false>(a, p.dt, stream);
  return p.causal ? launch_fwd_t<64, true>(a, p.dt, stream) : launch_fwd_t<64, false>(a, p.dt, stream);
}

hipError_t launch_attn_bwd(const AttnProblem& p, hipStream_t stream) {
  AttnBwdArgs a{};
  a.qkv = p.qkv;
  a.o = p.o;
  a.dout = p.dout;
  a.lse = p.lse;
  a.delta = p.delta;
  a.dqkv = p.dqkv;
  a.s = p.s;
  a.b = p.b;
  a.nh = p.nh;
  a.T = p.T;
  a.nqb = (p.s + AQ - 1) / AQ;
  a.scale = 1.0f / sqrtf(static_cast<float>(p.dh));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.qkv_shard_bytes = static_cast<uint32_t>(static_cast<int64_t>(p.s) * p.b * p.nh * 3 * p.dh * 2);
  a.o_shard_bytes = static_cast<uint32_t>(static_cast<int64_t>(p.s) * p.b * p.nh * p.dh * 2);
  a.mask = p.mask;
  a.mw = (p.s + 31) / 32;
  if (p.dh == 128)
    return p.causal ? launch_bwd_t<128, true>(a, p.dt, stream) : launch_bwd_t<128, false>(a, p.dt, stream);
  return p.causal ? launch_bwd_t<64, true>(a, p.dt, stream) : launch_bwd_t<64, false>(a, p.dt, stream);
}

}  // namespace tpmlp
