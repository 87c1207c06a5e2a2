// bf16 GEMM core for gfx950: C[M,N] = A[M,K]·B[K,N] with fp32 accumulation on
// the matrix cores (v_mfma_f32_32x32x16_bf16), batched over resident shards.
//
// Each of the six products of the tensor-parallel MLP shard is one instance
// ([TUT] §二: Z_i = X·A_i, P_i = Y_i·B_i, E_i = G·B_iᵀ, dA_i = Xᵀ·D_i,
// dB_i = Y_iᵀ·G, dX_i = D_i·A_iᵀ).  They differ only in operand storage order
// and in what the epilogue writes:
//   K-major operands are staged row by row and read with ds_read_b128;
//   M/N-major operands are staged as they lie in memory and read with the
//   gfx950 transposing LDS read (ds_read_b64_tr_b16), so no operand is ever
//   transposed in HBM.
//
// Tiling: 256×256 macro tile, K step 64, 4 waves (2×2), each wave owning a
// 128×128 sub-tile as 4×4 MFMA blocks of 32×32 (256 fp32 accumulators per
// lane, held in AGPRs).  Global→LDS traffic uses buffer_load … lds (16 B per
// lane) into two LDS stages (2 × 64 KiB); edges are zero-filled by the buffer
// descriptor's range check, so one code path serves every shape.  One
// workgroup barrier per K step: it both publishes the next stage and frees the
// current one.
//
// LDS fragment reads are issued as inline asm with explicit lgkmcnt waits that
// carry the fragment registers as operands, so (a) reads for the next 16-wide
// K slice are in flight while the current slice's 16 MFMAs run, and (b) the
// compiler's conservative "wait for every LDS DMA" before a transposing read
// is never inserted (the DMA completion is awaited once per stage, before the
// barrier).
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int OP_TILE_BYTES = 256 * BK * 2;  // one operand tile, 32 KiB
constexpr int STAGE_BYTES = 2 * OP_TILE_BYTES;
constexpr uint32_t OOB = 0x80000000u;  // past every descriptor's range (< 2^31)

struct KArgs {
  const bf16* A;
  const bf16* B;
  void* C;
  void* C2;
  const bf16* Zin;
  int M, N, K;
  int tiles_m, tiles_n, batch;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;
  uint32_t a_bytes, b_bytes;
};

// ---------------------------------------------------------------------------
// LDS tile layouts (one 256-row × 64-k operand tile = 32 KiB).
//
// KMAJ: [256 rows][64 k], 128 B per row.  The 16-B chunk c (8 k values) of
//   row r sits at chunk slot c ^ (r & 7): the 8 lanes that read one chunk of 8
//   consecutive rows hit 8 different bank groups.
// MNMAJ: [8 column blocks][64 k][32 columns], 64 B per (block, k) row.  Chunk
//   c (0..3) of k-row k sits at slot c ^ (((k >> 1) & 1) << 1): a 16-lane
//   transposing read of 4 consecutive k-rows × 32 B then covers the 8 distinct
//   16-B slots of a 128-B bank line.
// ---------------------------------------------------------------------------

template <int ORDER>
__device__ __forceinline__ void issue_tile(i32x4 rsrc, TPMLP_LDS char* tile, int r0, int k0, int R,
                                           int K, int64_t ld, int wave, int lane) {
  if constexpr (ORDER == KMAJ) {
    // 8 instructions per wave, each 8 rows × 128 B.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = wave * 64 + j * 8 + (lane >> 3);
      const int c = (lane & 7) ^ (lane >> 3);  // row & 7 == lane >> 3
      const int gr = r0 + row, gk = k0 + c * 8;
      const bool ok = gr < R && gk < K;
      const uint32_t voff =
          ok ? static_cast<uint32_t>((static_cast<int64_t>(gr) * ld + gk) * 2) : OOB;
      buffer_load_lds16(rsrc, tile + (wave * 64 + j * 8) * 128, voff);
    }
  } else {
    // 8 instructions per wave, each one column block × 16 k-rows × 64 B.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int seg = wave * 8 + j;  // 32 segments of 1 KiB
      const int blk = seg >> 2;      // column block 0..7
      const int kr = (seg & 3) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ (((kr >> 1) & 1) << 1);
      const int gk = k0 + kr, gr = r0 + blk * 32 + c * 8;
      const bool ok = gk < K && gr < R;
      const uint32_t voff =
          ok ? static_cast<uint32_t>((static_cast<int64_t>(gk) * ld + gr) * 2) : OOB;
      buffer_load_lds16(rsrc, tile + seg * 1024, voff);
    }
  }
}

// Per-lane LDS byte offsets (relative to the operand tile) of the fragment
// reads.  A fragment covers 32 rows (of M or N) × one 16-wide K slice; lane L
// receives row L%32, k = 8·(L/32) + 0..7 of the slice.
struct FragAddr {
  uint32_t a[4];  // KMAJ: one base per K slice; MNMAJ: a[0] only
};

template <int ORDER>
__device__ __forceinline__ FragAddr frag_addr(int rbase, int lane) {
  FragAddr f;
  if constexpr (ORDER == KMAJ) {
    const int rr = rbase + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      f.a[ks] = rr * 128 + ((c ^ (rr & 7)) << 4);
    }
  } else {
    // ds_read_b64_tr_b16: in each 16-lane group, lane i reads 4 elements of
    // k-row i/4, columns 4·(i%4)..+3 of a 4×16 block; after the transpose
    // lane i holds column i of the block for k-rows 0..3.  Groups: g&1 picks
    // columns 0-15 / 16-31 of the fragment, g>>1 picks k 0-7 / 8-15.
    const int g = lane >> 4, i = lane & 15;
    const int col = (g & 1) * 16 + (i & 3) * 4;  // within the 32-column block
    const int kq = (g >> 1) * 8 + (i >> 2);
    const int c = (col >> 3) ^ (((kq >> 1) & 1) << 1);
    f.a[0] = (rbase >> 5) * 4096 + kq * 64 + (c << 4) + (col & 7) * 2;
    f.a[1] = f.a[2] = f.a[3] = 0;
  }
  return f;
}

#define TPMLP_DS_READ_B128(dst, addr, OFF) \
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF))
#define TPMLP_DS_READ_TR(dst, addr, OFF) \
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF))

typedef int i32x2 __attribute__((ext_vector_type(2)));

// Issue the 4 fragment reads of one operand for K slice KS.  TILE_OFF is the
// operand tile's byte offset inside the stage; `base` already includes the
// stage offset.
template <int ORDER, int KS, int TILE_OFF>
__device__ __forceinline__ void read_frags(i32x4 (&fr)[4], const FragAddr& fa, uint32_t stage) {
  if constexpr (ORDER == KMAJ) {
    const uint32_t a = fa.a[KS] + stage;
    TPMLP_DS_READ_B128(fr[0], a, TILE_OFF + 0 * 4096);
    TPMLP_DS_READ_B128(fr[1], a, TILE_OFF + 1 * 4096);
    TPMLP_DS_READ_B128(fr[2], a, TILE_OFF + 2 * 4096);
    TPMLP_DS_READ_B128(fr[3], a, TILE_OFF + 3 * 4096);
  } else {
    const uint32_t a = fa.a[0] + stage;
    i32x2 lo[4], hi[4];
    TPMLP_DS_READ_TR(lo[0], a, TILE_OFF + 0 * 4096 + KS * 1024);
    TPMLP_DS_READ_TR(hi[0], a, TILE_OFF + 0 * 4096 + KS * 1024 + 256);
    TPMLP_DS_READ_TR(lo[1], a, TILE_OFF + 1 * 4096 + KS * 1024);
    TPMLP_DS_READ_TR(hi[1], a, TILE_OFF + 1 * 4096 + KS * 1024 + 256);
    TPMLP_DS_READ_TR(lo[2], a, TILE_OFF + 2 * 4096 + KS * 1024);
    TPMLP_DS_READ_TR(hi[2], a, TILE_OFF + 2 * 4096 + KS * 1024 + 256);
    TPMLP_DS_READ_TR(lo[3], a, TILE_OFF + 3 * 4096 + KS * 1024);
    TPMLP_DS_READ_TR(hi[3], a, TILE_OFF + 3 * 4096 + KS * 1024 + 256);
#pragma unroll
    for (int q = 0; q < 4; ++q) fr[q] = __builtin_shufflevector(lo[q], hi[q], 0, 1, 2, 3);
  }
}

template <int ORDER>
constexpr int reads_per_operand() {
  return ORDER == KMAJ ? 4 : 8;
}

// Wait until at most N LDS reads are outstanding; the fragment registers are
// in/out operands so no use of them can be scheduled above the wait.
template <int N>
__device__ __forceinline__ void wait_frags(i32x4 (&a)[4], i32x4 (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                 "+v"(b[2]), "+v"(b[3])
               : "i"(N));
}

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void mma16(f32x16 (&acc)[4][4], const i32x4 (&a)[4], const i32x4 (&b)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(b[j]),
                                                          acc[i][j], 0, 0, 0);
}

// Map the linear workgroup id to a tile so that the tiles one XCD works on
// form one contiguous range (workgroups are dealt to the 8 XCDs round-robin;
// each XCD has its own L2).
__device__ __forceinline__ int xcd_tile(int wg, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = wg & 7, local = wg >> 3;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

template <int AO, int BO, int EPI>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(KArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
  TPMLP_LDS char* lds = (TPMLP_LDS char*)(smem);
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  const int per_batch = a.tiles_m * a.tiles_n;
  const int tile = xcd_tile(blockIdx.x, per_batch * a.batch);
  const int batch = tile / per_batch;
  const int t2 = tile - batch * per_batch;
  const int tm = t2 / a.tiles_n, tn = t2 - (t2 / a.tiles_n) * a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const i32x4 ra = make_rsrc(a.A + batch * a.sA, a.a_bytes);
  const i32x4 rb = make_rsrc(a.B + batch * a.sB, a.b_bytes);

  const FragAddr fa = frag_addr<AO>(wm * 128, lane);
  const FragAddr fb = frag_addr<BO>(wn * 128, lane);
  constexpr int NR = reads_per_operand<AO>() + reads_per_operand<BO>();
  constexpr int NRW = NR > 15 ? 15 : NR;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int KT = (a.K + BK - 1) / BK;
  if (KT > 0) {
    issue_tile<AO>(ra, lds, m0, 0, a.M, a.K, a.lda, wave, lane);
    issue_tile<BO>(rb, lds + OP_TILE_BYTES, n0, 0, a.N, a.K, a.ldb, wave, lane);
    wait_vmcnt<0>();
    block_barrier();
  }
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) {
      TPMLP_LDS char* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
      issue_tile<AO>(ra, nxt, m0, (kt + 1) * BK, a.M, a.K, a.lda, wave, lane);
      issue_tile<BO>(rb, nxt + OP_TILE_BYTES, n0, (kt + 1) * BK, a.N, a.K, a.ldb, wave, lane);
    }
    const uint32_t st = lds_base + (kt & 1) * STAGE_BYTES;
    i32x4 a0[4], b0[4], a1[4], b1[4];
    read_frags<AO, 0, 0>(a0, fa, st);
    read_frags<BO, 0, OP_TILE_BYTES>(b0, fb, st);
    read_frags<AO, 1, 0>(a1, fa, st);
    read_frags<BO, 1, OP_TILE_BYTES>(b1, fb, st);
    wait_frags<NRW>(a0, b0);
    mma16(acc, a0, b0);
    read_frags<AO, 2, 0>(a0, fa, st);
    read_frags<BO, 2, OP_TILE_BYTES>(b0, fb, st);
    wait_frags<NRW>(a1, b1);
    mma16(acc, a1, b1);
    read_frags<AO, 3, 0>(a1, fa, st);
    read_frags<BO, 3, OP_TILE_BYTES>(b1, fb, st);
    wait_frags<NRW>(a0, b0);
    mma16(acc, a0, b0);
    wait_frags<0>(a1, b1);
    mma16(acc, a1, b1);
    // The next stage's loads have landed (this wave's share) and this wave is
    // done reading the current stage; the barrier makes both hold for all.
    wait_vmcnt<0>();
    block_barrier();
  }

  // Epilogue.  32×32 block (i, j), accumulator v of lane L holds
  // row 8·(v/4) + 4·(L/32) + v%4, column L%32.
  const int64_t cb = static_cast<int64_t>(batch) * a.sC;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
      if (col >= a.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (row >= a.M) continue;
        const int64_t off = cb + static_cast<int64_t>(row) * a.ldc + col;
        const float x = acc[i][j][v];
        if constexpr (EPI == EPI_STORE) {
          static_cast<bf16*>(a.C)[off] = f2bf(x);
        } else if constexpr (EPI == EPI_STORE_F32) {
          static_cast<float*>(a.C)[off] = x;
        } else if constexpr (EPI == EPI_GELU_ZY) {
          static_cast<bf16*>(a.C)[off] = f2bf(x);
          static_cast<bf16*>(a.C2)[off] = f2bf(gelu_fast(x));
        } else {
          const float z = bf2f(a.Zin[off]);
          static_cast<bf16*>(a.C)[off] = f2bf(x * gelu_grad_fast(z));
        }
      }
    }
  }
}

template <int AO, int BO, int EPI>
hipError_t launch_t(const KArgs& k, hipStream_t stream) {
  dim3 grid(k.tiles_m * k.tiles_n * k.batch);
  hipLaunchKernelGGL((gemm_bf16_kernel<AO, BO, EPI>), grid, dim3(NTHR), 0, stream, k);
  return hipGetLastError();
}

uint32_t extent_bytes(int order, int rows, int K, int64_t ld) {
  // bytes spanned by a rows×K operand of the given storage order
  if (rows <= 0 || K <= 0) return 0;
  int64_t elems = order == KMAJ ? (static_cast<int64_t>(rows) - 1) * ld + K
                                : (static_cast<int64_t>(K) - 1) * ld + rows;
  return static_cast<uint32_t>(elems * 2);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmProblem& p, int a_order, int b_order, int epi,
                            hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
  KArgs k;
  k.A = static_cast<const bf16*>(p.A);
  k.B = static_cast<const bf16*>(p.B);
  k.C = p.C;
  k.C2 = p.C2;
  k.Zin = static_cast<const bf16*>(p.Zin);
  k.M = p.M;
  k.N = p.N;
  k.K = p.K;
  k.tiles_m = (p.M + BM - 1) / BM;
  k.tiles_n = (p.N + BN - 1) / BN;
  k.batch = p.batch;
  k.lda = p.lda;
  k.ldb = p.ldb;
  k.ldc = p.ldc;
  k.sA = p.sA;
  k.sB = p.sB;
  k.sC = p.sC;
  k.a_bytes = extent_bytes(a_order, p.M, p.K, p.lda);
  k.b_bytes = extent_bytes(b_order, p.N, p.K, p.ldb);
  if (a_order == KMAJ && b_order == MNMAJ && epi == EPI_GELU_ZY)
    return launch_t<KMAJ, MNMAJ, EPI_GELU_ZY>(k, stream);
  if (a_order == KMAJ && b_order == MNMAJ && epi == EPI_STORE)
    return launch_t<KMAJ, MNMAJ, EPI_STORE>(k, stream);
  if (a_order == KMAJ && b_order == KMAJ && epi == EPI_GELU_GRAD)
    return launch_t<KMAJ, KMAJ, EPI_GELU_GRAD>(k, stream);
  if (a_order == KMAJ && b_order == KMAJ && epi == EPI_STORE)
    return launch_t<KMAJ, KMAJ, EPI_STORE>(k, stream);
  if (a_order == MNMAJ && b_order == MNMAJ && epi == EPI_STORE_F32)
    return launch_t<MNMAJ, MNMAJ, EPI_STORE_F32>(k, stream);
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
