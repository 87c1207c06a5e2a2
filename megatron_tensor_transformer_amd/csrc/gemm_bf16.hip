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
// Tiling: 256×256 macro tile, K step 64, 8 waves (2×4), each wave owning a
// 128×64 sub-tile as 4×2 MFMA blocks of 32×32 (128 fp32 accumulators per
// lane, in AGPRs).  Two waves share each SIMD, so when one waits (an LDS read,
// a DMA issue held up by a full address queue, the barrier) the other keeps
// the matrix core busy.  The B fragment is the MFMA's first operand, so each
// lane ends up holding 4 consecutive output columns of one row.
//
// Global→LDS: buffer_load … lds (16 B per lane; edges zero-filled by the
// buffer descriptor's range check, so one code path serves every shape).  The
// A operand has 3 LDS stages and is fetched two K steps ahead, the B operand
// has 2 stages and is fetched one step ahead: 5 × 32 KiB = all 160 KiB of LDS.
// One workgroup barrier per K step publishes the stages that just landed and
// frees the ones just consumed.
//
// The K-step body is a fixed interleaving written as inline asm, so that the
// compiler keeps it: the 32 MFMAs of a wave's step are each followed by at most
// a fragment read for the next 16-wide K slice and a DMA load for a later
// step, so memory instructions never come in bursts.  Fragment registers are
// double-buffered across K slices; the lgkmcnt waits carry them as operands.
//
// Epilogue: bf16 outputs are staged through LDS (each wave its own 128×64
// region) and written with coalesced 16-B stores; fp32 outputs are written
// straight from the accumulators as 16-B stores.
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "tile_map.h"

namespace tpmlp {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NWAVE = 8, NTHR = NWAVE * 64;
constexpr int FA = 4, FB = 2;           // 32-row fragments per wave: 128 rows of A, 64 columns of B
constexpr int NLOAD = 32 / NWAVE;      // 1-KiB DMA loads per wave per operand stage
constexpr int TILE_BYTES = 256 * BK * 2;  // one operand stage, 32 KiB
constexpr int A_STAGES = 3, B_STAGES = 2;
constexpr int B_BASE = A_STAGES * TILE_BYTES;
constexpr int LDS_BYTES = (A_STAGES + B_STAGES) * TILE_BYTES;  // 160 KiB
constexpr uint32_t OOB = 0x80000000u;  // past every descriptor's range (< 2^31)

struct alignas(64) KArgs {
  const bf16* A;
  const bf16* B;
  void* C;
  void* C2;
  const bf16* Zin;
  const bf16* bias;
  int64_t sBias;
  float* rstats;
  float* colsum;
  int M, N, K;
  int tiles_m, tiles_n, batch;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;
  uint32_t a_bytes, b_bytes, c_bytes;
  // split K: ksplit slices of kchunk (a multiple of BK) each; slice s writes
  // its fp32 partial tile at C + s·sSlice (ksplit = 1: no split)
  int ksplit, kchunk;
  int64_t sSlice;
  // K-split tail (sk_L > 0: this problem's work items are tail pieces): the
  // sk_T tiles from tile index sk_first on (sk_KS K steps each) each split
  // into sk_q pieces of sk_L steps; item c = j·sk_T + u takes steps
  // [j·sk_L, min((j+1)·sk_L, sk_KS)) of tail tile u and writes its fp32
  // partial into slot c of sk_ws (256×256 floats per slot).  Items with the
  // same j cover the same K range, so neighbouring tiles' items share their
  // operand slices in the L2.
  int sk_L, sk_T, sk_first, sk_KS, sk_q;
  float* sk_ws;
};

// One launch runs up to three problems: p[0] and p[1] (the long group, one
// kind of operand orders and epilogue) and p[2] (another kind or the same);
// t0..t2 are their tile counts (zero for an absent problem).
struct KGroup {
  KArgs p[3];
  int t0, t1, t2;
  XcdSplit split;  // the order of the tiles over the XCDs (tile_map.h)
};

typedef int i32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// LDS operand tile layouts (256 rows of M or N × 64 k = 32 KiB).
//
// KMAJ: [256 rows][64 k], 128 B per row.  Chunk c (8 k values) of row r sits
//   at chunk slot c ^ ((r >> 1) & 7).  The LDS serves 256 B per clock (64
//   banks), i.e. 16 lanes of a 16-B read: those lanes read one chunk of 16
//   consecutive rows, even rows in one 128-B half of the bank line and odd rows
//   in the other, and the swizzle gives the 8 rows of each half 8 slots.
// MNMAJ: [8 column blocks][64 k][32 columns], 64 B per (block, k) row.  Chunk
//   c (0..3) of k-row k sits at slot c ^ (((k >> 1) & 1) << 1): the 32 lanes
//   of two 16-lane transposing reads then cover 4 k-rows × 64 B = 256 B once.
// ---------------------------------------------------------------------------

// Per-lane DMA offsets for one operand: the NLOAD loads a wave issues per
// stage.  base[j] is the byte offset of the lane's 16-B chunk at k0 = 0 (OOB
// when the row lies past the matrix edge); the k part is added per step.
// kq / kq_odd are the lane's k offset inside the step, for the K-edge test.
template <int NL = NLOAD>
struct LoadPlan {
  uint32_t base[NL];
  uint32_t kstep;  // bytes to add per K step (64 k)
  int kq;
  int kq_odd;
  int kseg;        // NL odd, M/N-major: 16·((NL·wave) % 4), the k-rows of load 0
};

// NL loads per wave and stage: 4 for a 256-row operand stage, 3 for a
// 192-row one (the B stage of the 256×192 tile).
template <int ORDER, int NL = NLOAD>
__device__ __forceinline__ LoadPlan<NL> make_plan(int r0, int R, int64_t ld, int wave, int lane) {
  LoadPlan<NL> p;
  p.kseg = 0;
  if constexpr (ORDER == KMAJ) {
    // load j: rows (NL·wave + j)·8 .. +7; lane: row + lane/8, slot lane%8
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int row = (wave * NL + j) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      const int gr = r0 + row;
      p.base[j] = gr < R ? static_cast<uint32_t>((static_cast<int64_t>(gr) * ld + c * 8) * 2) : OOB;
    }
    p.kstep = BK * 2;
    // (row >> 1) & 7 = (4·(NL·wave + j) + lane/16) & 7 only depends on the
    // parity of NL·wave + j: of j when NL is even; for odd NL the two values
    // trade places on odd waves, so that the parity of j still picks
    p.kq = ((lane & 7) ^ ((lane >> 4) & 7)) * 8;
    p.kq_odd = ((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 8;
    if constexpr (NL & 1) {
      if (wave & 1) {
        const int t = p.kq;
        p.kq = p.kq_odd;
        p.kq_odd = t;
      }
    }
  } else {
    // load j: column block seg/4, k-rows 16·(seg%4) + lane/4, seg = NL·wave + j
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int seg = wave * NL + j;
      const int blk = seg >> 2;
      const int kr = (seg & 3) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ (((kr >> 1) & 1) << 1);
      const int gr = r0 + blk * 32 + c * 8;
      p.base[j] = gr < R ? static_cast<uint32_t>((static_cast<int64_t>(kr) * ld + gr) * 2) : OOB;
    }
    p.kstep = static_cast<uint32_t>(BK * ld * 2);
    p.kq = lane >> 2;
    p.kq_odd = 0;
    if constexpr (NL & 3) p.kseg = ((NL * wave) & 3) * 16;
  }
  return p;
}

// DMA load J of one operand for the K step at byte offset koff (krem = K minus
// the step's first k) into stage `tile`.
template <int ORDER, int J, int NL = NLOAD>
__device__ __forceinline__ void dma(i32x4 rsrc, TPMLP_LDS char* tile, const LoadPlan<NL>& p, uint32_t koff,
                                    int krem, int wave) {
  bool ok;
  if constexpr (ORDER == KMAJ)
    ok = ((J & 1) ? p.kq_odd : p.kq) < krem;
  else if constexpr ((NL & 3) == 0)
    ok = (J & 3) * 16 + p.kq < krem;
  else
    ok = ((p.kseg + J * 16) & 63) + p.kq < krem;
  const uint32_t voff = ok ? p.base[J] + koff : OOB;
  // both layouts: load (NL·wave + J) fills the tile's 1-KiB segment of that
  // index; the LDS destination (M0) from a scalar copy of the uniform wave index
  const int ws = __builtin_amdgcn_readfirstlane(wave);
  buffer_load_lds16(rsrc, tile + (ws * NL + J) * 1024, voff);
}

template <int ORDER, int NL = NLOAD, int J = 0>
__device__ __forceinline__ void dma_all(i32x4 rsrc, TPMLP_LDS char* tile, const LoadPlan<NL>& p, uint32_t koff,
                                        int krem, int wave) {
  if constexpr (J < NL) {
    dma<ORDER, J, NL>(rsrc, tile, p, koff, krem, wave);
    dma_all<ORDER, NL, J + 1>(rsrc, tile, p, koff, krem, wave);
  }
}

// Per-lane LDS byte offsets of the fragment reads (relative to a stage).  A
// fragment covers 32 rows (of M or N) × one 16-wide K slice; lane L receives
// row L%32, k = 8·(L/32) + 0..7 of the slice.
template <int ORDER>
__device__ __forceinline__ void frag_addr(uint32_t (&f)[4], int rbase, int lane) {
  if constexpr (ORDER == KMAJ) {
    const int rr = rbase + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      f[ks] = rr * 128 + ((c ^ ((rr >> 1) & 7)) << 4);
    }
  } else {
    // ds_read_b64_tr_b16: in each 16-lane group, lane i reads 4 elements of
    // k-row i/4, columns 4·(i%4)..+3 of a 4×16 block; after the transpose
    // lane i holds column i of the block for k-rows 0..3.  Groups: g&1 picks
    // columns 0-15 / 16-31 of the fragment, g>>1 picks k 0-7 / 8-15.
    const int g = lane >> 4, i = lane & 15;
    const int col = (g & 1) * 16 + (i & 3) * 4;
    const int kq = (g >> 1) * 8 + (i >> 2);
    const int c = (col >> 3) ^ (((kq >> 1) & 1) << 1);
    f[0] = (rbase >> 5) * 4096 + kq * 64 + (c << 4) + (col & 7) * 2;
    f[1] = f[2] = f[3] = 0;
  }
}

// LDS read instructions per K slice for NF fragments
template <int ORDER, int NF>
constexpr int reads_per_slice() {
  return ORDER == KMAJ ? NF : 2 * NF;
}

// Read op T of one operand for K slice KS.  KMAJ: op T is fragment T.  MNMAJ:
// op T is half T&1 (k 0-3 / 4-7 of the lane's 8) of fragment T>>1.
template <int ORDER, int KS, int T, int NF>
__device__ __forceinline__ void read_op(i32x4 (&fr)[NF], const uint32_t (&f)[4], uint32_t stage) {
  if constexpr (ORDER == KMAJ) {
    const uint32_t a = f[KS] + stage;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fr[T]) : "v"(a), "i"(T * 4096));
  } else {
    const uint32_t a = f[0] + stage;
    i32x2 h;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(h)
                 : "v"(a), "i"((T >> 1) * 4096 + KS * 1024 + (T & 1) * 256));
    if constexpr (T & 1) {
      fr[T >> 1][2] = h[0];
      fr[T >> 1][3] = h[1];
    } else {
      fr[T >> 1][0] = h[0];
      fr[T >> 1][1] = h[1];
    }
  }
}

// Wait until no LDS read is outstanding; the fragment registers are in/out
// operands so no use of them can be placed above the wait.
__device__ __forceinline__ void wait_frags(i32x4 (&a)[FA], i32x4 (&b)[FB]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]));
}
// the same for the 256×192 tile's fragments (2 of A, 3 of B) and the
// 256×128 tile's (2 and 2)
__device__ __forceinline__ void wait_frags(i32x4 (&a)[2], i32x4 (&b)[3]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]));
}
__device__ __forceinline__ void wait_frags(i32x4 (&a)[2], i32x4 (&b)[2]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]));
}

#define TPMLP_MFMA(ACC, BF, AF) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(ACC) : "v"(BF), "v"(AF))

template <int FA_ = FA, int FB_ = FB>
constexpr int n_reads(int ao, int bo) {
  return (ao == KMAJ ? FA_ : 2 * FA_) + (bo == KMAJ ? FB_ : 2 * FB_);
}

// One read op for the next slice, from the merged A-then-B op list.
template <int AO, int BO, int KS, int T, int FA_ = FA, int FB_ = FB>
__device__ __forceinline__ void next_read(i32x4 (&fa)[FA_], i32x4 (&fb)[FB_], const uint32_t (&pa)[4],
                                          const uint32_t (&pb)[4], uint32_t sa, uint32_t sb) {
  constexpr int NA = reads_per_slice<AO, FA_>();
  if constexpr (T < NA)
    read_op<AO, KS, T>(fa, pa, sa);
  else
    read_op<BO, KS, T - NA>(fb, pb, sb);
}

template <int AO, int BO, int KS, int FA_ = FA, int FB_ = FB, int T = 0>
__device__ __forceinline__ void read_slice(i32x4 (&fa)[FA_], i32x4 (&fb)[FB_], const uint32_t (&pa)[4],
                                           const uint32_t (&pb)[4], uint32_t sa, uint32_t sb) {
  if constexpr (T < n_reads<FA_, FB_>(AO, BO)) {
    next_read<AO, BO, KS, T, FA_, FB_>(fa, fb, pa, pb, sa, sb);
    read_slice<AO, BO, KS, FA_, FB_, T + 1>(fa, fb, pa, pb, sa, sb);
  }
}

struct StepCtx {
  i32x4 rA, rB;
  TPMLP_LDS char* dA;
  TPMLP_LDS char* dB;
  uint32_t sa, sb;    // this step's A and B stages
  uint32_t nsa, nsb;  // the next step's
  uint32_t koA, koB;
  int kremA, kremB, wave;
};

// The FA·FB MFMAs of slice S (8 for the 256×256 tile, 6 for 256×192, 4 for
// 256×128).  After MFMA Q come the next slice's reads Q and Q + FA·FB (for
// S = 3, slice 0 of the next step, from its stages) and, at odd Q, one DMA
// load: of A two steps ahead in slice 1 (and, when slice 1 has fewer odd
// slots than A has loads, in slice 2), of B two steps ahead in slice 3.
template <int AO, int BO, int S, int FA_ = FA, int FB_ = FB, int NLB = NLOAD, int Q = 0>
__device__ __forceinline__ void slice_body(f32x16 (&acc)[FA_][FB_], i32x4 (&ca)[FA_], i32x4 (&cb)[FB_],
                                           i32x4 (&na)[FA_], i32x4 (&nb)[FB_], const uint32_t (&pa)[4],
                                           const uint32_t (&pb)[4], const LoadPlan<NLOAD>& la,
                                           const LoadPlan<NLB>& lb, const StepCtx& s) {
  constexpr int NQ = FA_ * FB_;
  if constexpr (Q < NQ) {
    TPMLP_MFMA(acc[Q / FB_][Q % FB_], cb[Q % FB_], ca[Q / FB_]);
    constexpr int NR = n_reads<FA_, FB_>(AO, BO);
    if constexpr (S < 3 && Q < NR) next_read<AO, BO, S + 1, Q, FA_, FB_>(na, nb, pa, pb, s.sa, s.sb);
    if constexpr (S == 3 && Q < NR) next_read<AO, BO, 0, Q, FA_, FB_>(na, nb, pa, pb, s.nsa, s.nsb);
    if constexpr (S < 3 && Q + NQ < NR) next_read<AO, BO, S + 1, Q + NQ, FA_, FB_>(na, nb, pa, pb, s.sa, s.sb);
    if constexpr (S == 3 && Q + NQ < NR) next_read<AO, BO, 0, Q + NQ, FA_, FB_>(na, nb, pa, pb, s.nsa, s.nsb);
    if constexpr (S == 1 && (Q & 1) && (Q >> 1) < NLOAD)
      dma<AO, (Q >> 1)>(s.rA, s.dA, la, s.koA, s.kremA, s.wave);
    if constexpr (S == 2 && (Q & 1) && NQ / 2 + (Q >> 1) < NLOAD)
      dma<AO, NQ / 2 + (Q >> 1)>(s.rA, s.dA, la, s.koA, s.kremA, s.wave);
    if constexpr (S == 3 && (Q & 1) && (Q >> 1) < NLB)
      dma<BO, (Q >> 1), NLB>(s.rB, s.dB, lb, s.koB, s.kremB, s.wave);
    slice_body<AO, BO, S, FA_, FB_, NLB, Q + 1>(acc, ca, cb, na, nb, pa, pb, la, lb, s);
  }
}

// Within a problem's batch the tiles go in groups of GM tile rows, so the
// workgroups resident on one XCD share operand panels in its L2 (the order of
// tiles over the XCDs is in tile_map.h).
__device__ __forceinline__ void tile_coords(int tile, const KArgs& a, int& batch, int& tm, int& tn) {
  const int per_batch = a.tiles_m * a.tiles_n;
  batch = tile / per_batch;
  const int t2 = tile - batch * per_batch;
  constexpr int GM = 4;
  const int grp = t2 / (GM * a.tiles_n);
  const int fm = grp * GM;
  const int gm = a.tiles_m - fm < GM ? a.tiles_m - fm : GM;
  const int rem = t2 - grp * GM * a.tiles_n;
  tm = fm + rem % gm;
  tn = rem / gm;
}

__device__ __forceinline__ i32x2 pack4_bf16(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = f2bf(a);
  v[1] = f2bf(b);
  v[2] = f2bf(c);
  v[3] = f2bf(d);
  return __builtin_bit_cast(i32x2, v);
}

// Epilogue staging region (per wave, 128 rows × 64 columns of bf16, 128 B per
// row): chunk c (8 columns) of row r sits at slot c ^ (r & 7).
constexpr int QROW = 128, QBYTES = 128 * QROW;
static_assert(NWAVE * (QBYTES + 128) <= LDS_BYTES, "epilogue staging and bias exceed the LDS");
// fp32 staging (half a wave's region at a time): 64 rows × 64 floats
constexpr int FQROW = 256, FQBYTES = 64 * FQROW;
static_assert(NWAVE * FQBYTES <= LDS_BYTES, "fp32 epilogue staging exceeds the LDS");
// 16-B chunk slot of a staging row.  A row is 128 B, half of the LDS's 256-B
// bank width, so rows of one parity share a bank half; XOR-ing with row/2
// gives the 16 rows of a parity that one accumulator write covers 8 distinct
// slots (2 rows per bank: the minimum for 512 B), and a 1-KB read of 8 whole
// rows touches each bank 4 times (also the minimum).
__device__ __forceinline__ int quad_slot(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ uint32_t quad_addr(uint32_t qbase, int row, int chunk, int half) {
  return qbase + row * QROW + (quad_slot(row, chunk) << 4) + half * 8;
}

// The 256×192 and 256×128 tiles' epilogue (defined below).
template <int EPI, int TN>
__device__ void epilogue_narrow(const KArgs& a, f32x16 (&acc)[2][TN / 64], int batch, int m0, int n0,
                                TPMLP_LDS char* lds);

// One output tile of problem a: 256×TN, TN = 256 (8 waves as 2×4, each 128×64:
// 4×2 blocks), TN = 192 (8 waves as 4×2, each 64×96: 2×3 blocks; its B
// stage holds 192 rows and takes 3 DMA loads per wave) or TN = 128 (4×2
// waves of 64×64: 2×2 blocks; 2 B loads per wave).
template <int AO, int BO, int EPI, int TN = BN>
__device__ __forceinline__ void gemm_tile(const KArgs& a, int tile, TPMLP_LDS char* lds) {
  static_assert(TN == 256 || TN == 192 || TN == 128, "tile width");
  constexpr int FA_ = TN == 256 ? FA : 2, FB_ = TN == 256 ? FB : TN / 64;
  constexpr int WN = TN / (32 * FB_);   // waves across N: 4 or 2
  constexpr int NLB = TN / 64;          // B loads per wave and stage: 4 or 3
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  int batch, tm, tn;
  tile_coords(tile, a, batch, tm, tn);
  const int m0 = tm * BM, n0 = tn * TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const i32x4 rA = make_rsrc(a.A + batch * a.sA, a.a_bytes);
  const i32x4 rB = make_rsrc(a.B + batch * a.sB, a.b_bytes);
  const LoadPlan<NLOAD> la = make_plan<AO>(m0, a.M, a.lda, wave, lane);
  const LoadPlan<NLB> lb = make_plan<BO, NLB>(n0, a.N, a.ldb, wave, lane);
  uint32_t pa[4], pb[4];
  frag_addr<AO>(pa, wm * 32 * FA_, lane);
  frag_addr<BO>(pb, wn * 32 * FB_, lane);

  f32x16 acc[FA_][FB_];
#pragma unroll
  for (int i = 0; i < FA_; ++i)
#pragma unroll
    for (int j = 0; j < FB_; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int KT = (a.K + BK - 1) / BK;
  // Stages: A is triple-buffered (step kt in A stage kt % 3), B double-buffered
  // (B stage kt % 2).  The DMA loads run two steps ahead: A(kt+2) is issued in
  // slice 1 of step kt, into the stage step kt-1 used; B(kt+2) in slice 3 of
  // step kt, into the stage step kt used.  Each step has one barrier, between
  // slices 2 and 3: every fragment of the step is in registers by then, so
  // the barrier both frees the step's stages and (after this wave's wait for
  // B(kt+1), A(kt+1)) publishes the next step's, whose slice 0 is read while
  // slice 3's MFMAs run.
  i32x4 fa0[FA_], fb0[FB_], fa1[FA_], fb1[FB_];
  if (KT > 0) {
    // prologue: A(0), B(0), A(1), B(1); wait for the first two
    dma_all<AO>(rA, lds, la, 0, a.K, wave);
    dma_all<BO, NLB>(rB, lds + B_BASE, lb, 0, a.K, wave);
    dma_all<AO>(rA, lds + TILE_BYTES, la, la.kstep, a.K - BK, wave);
    dma_all<BO, NLB>(rB, lds + B_BASE + TILE_BYTES, lb, lb.kstep, a.K - BK, wave);
    wait_vmcnt<NLOAD + NLB>();
    block_barrier();
    read_slice<AO, BO, 0, FA_, FB_>(fa0, fb0, pa, pb, lds_base, lds_base + B_BASE);
    wait_frags(fa0, fb0);
  }

  int sA = 0;  // A stage of step kt (= kt % 3)
  for (int kt = 0; kt < KT; ++kt) {
    const int sA1 = sA == 2 ? 0 : sA + 1;  // (kt + 1) % 3
    const int sA2 = sA == 0 ? 2 : sA - 1;  // (kt + 2) % 3
    StepCtx s;
    s.rA = rA;
    s.rB = rB;
    s.sa = lds_base + sA * TILE_BYTES;
    s.sb = lds_base + B_BASE + (kt & 1) * TILE_BYTES;
    s.nsa = lds_base + sA1 * TILE_BYTES;
    s.nsb = lds_base + B_BASE + ((kt + 1) & 1) * TILE_BYTES;
    s.dA = lds + sA2 * TILE_BYTES;
    s.dB = lds + B_BASE + (kt & 1) * TILE_BYTES;
    s.koA = static_cast<uint32_t>(kt + 2) * la.kstep;
    s.koB = static_cast<uint32_t>(kt + 2) * lb.kstep;
    s.kremA = a.K - (kt + 2) * BK;
    s.kremB = a.K - (kt + 2) * BK;
    s.wave = wave;

    slice_body<AO, BO, 0, FA_, FB_, NLB>(acc, fa0, fb0, fa1, fb1, pa, pb, la, lb, s);
    wait_frags(fa1, fb1);
    slice_body<AO, BO, 1, FA_, FB_, NLB>(acc, fa1, fb1, fa0, fb0, pa, pb, la, lb, s);
    wait_frags(fa0, fb0);
    slice_body<AO, BO, 2, FA_, FB_, NLB>(acc, fa0, fb0, fa1, fb1, pa, pb, la, lb, s);
    wait_frags(fa1, fb1);
    // B(kt+1) and A(kt+1) have landed (this wave's share); A(kt+2) may still
    // be in flight.
    wait_vmcnt<NLOAD>();
    block_barrier();
    slice_body<AO, BO, 3, FA_, FB_, NLB>(acc, fa1, fb1, fa0, fb0, pa, pb, la, lb, s);
    // the next step's slice-0 fragments (unused after the last step) must
    // have landed before their registers are touched again
    wait_frags(fa0, fb0);
    sA = sA1;
  }
  wait_vmcnt<0>();
  // The accumulators were last written by inline-asm MFMAs: give the MFMA
  // pipeline its passes before they are read.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ------------------------------------------------------------------ epilogue
  if constexpr (TN != BN) {
    epilogue_narrow<EPI, TN>(a, acc, batch, m0, n0, lds);
    return;
  } else {
  // Accumulator v of block (i, j) of lane L: row wm·128 + 32i + L%32,
  // columns wn·64 + 32j + 8·(v/4) + 4·(L/32) + v%4.
  const int row_l = lane & 31, half = lane >> 5;
  if constexpr (EPI == EPI_STORE_F32) {
    // fp32 results go through LDS as well: each wave stages half of its
    // 128×64 region at a time (64 rows × 256 B = 16 KiB; 8 waves use 128 KiB
    // of the main loop's stages), so that every store instruction writes 4
    // whole rows of 256 B, two full 128-B lines each, instead of 32 rows of
    // 32 B that fill their lines only in groups of four.  Chunk c (4 floats)
    // of staging row r sits at slot c ^ (r & 15): the 16 lanes that one LDS
    // cycle serves then hit 16 distinct slots, writing (16 rows, one chunk)
    // and reading (one row, 16 chunks) alike.
    block_barrier();  // every wave is done with the main-loop stages
    float* C = static_cast<float*>(a.C) + static_cast<int64_t>(batch) * a.sC;
    const uint32_t fbase = lds_base + wave * FQBYTES;
    const int qm0 = m0 + wm * 128, qn0 = n0 + wn * 64;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * hp + ii;
        const int r = ii * 32 + row_l;
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          float v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[i][j][e]));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = j * 8 + q * 2 + half;
            f32x4 w;
            w[0] = v[4 * q];
            w[1] = v[4 * q + 1];
            w[2] = v[4 * q + 2];
            w[3] = v[4 * q + 3];
            asm volatile("ds_write_b128 %0, %1" ::"v"(fbase + r * FQROW + ((c ^ (r & 15)) << 4)), "v"(w)
                         : "memory");
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it0 = 0; it0 < 16; it0 += 8) {
        f32x4 w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = (it0 + u) * 4 + (lane >> 4), c = lane & 15;
          asm volatile("ds_read_b128 %0, %1" : "=v"(w[u]) : "v"(fbase + r * FQROW + ((c ^ (r & 15)) << 4)) : "memory");
        }
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]), "+v"(w[6]),
                       "+v"(w[7])::"memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int gr = qm0 + 64 * hp + (it0 + u) * 4 + (lane >> 4), gc = qn0 + (lane & 15) * 4;
          if (gr < a.M && gc < a.N) *reinterpret_cast<f32x4*>(C + static_cast<int64_t>(gr) * a.ldc + gc) = w[u];
        }
      }
    }
  } else {
    block_barrier();  // every wave is done with the main-loop stages
    const uint32_t qbase = lds_base + wave * QBYTES;
    const int64_t cbase = static_cast<int64_t>(batch) * a.sC;
    const int qm0 = m0 + wm * 128, qn0 = n0 + wn * 64;
    constexpr bool ZY = EPI == EPI_GELU_ZY || EPI == EPI_BIAS_GELU_ZY;
    constexpr bool BIAS = EPI == EPI_BIAS_GELU_ZY || EPI == EPI_BIAS_STORE;
    constexpr int PASSES = ZY ? 2 : 1;
    // column bias (EPI_BIAS_GELU_ZY, EPI_BIAS_STORE): the wave's 64 bias values are staged
    // in LDS past the eight staging regions and read back per row block, so
    // they hold no registers across the passes (N is a multiple of 8, so a
    // 4-column group is inside N whenever its first column is)
    const uint32_t bbase = lds_base + NWAVE * QBYTES + wave * 128;
    if constexpr (BIAS) {
      if (lane < 16) {
        const int col = qn0 + lane * 4;
        const bf16* bias = a.bias + static_cast<int64_t>(batch) * a.sBias;
        const i32x2 b = col < a.N ? *reinterpret_cast<const i32x2*>(bias + col) : i32x2{0, 0};
        asm volatile("ds_write_b64 %0, %1" ::"v"(bbase + lane * 8), "v"(b) : "memory");
      }
    }

    constexpr bool GG = EPI == EPI_GELU_GRAD || EPI == EPI_GELU_GRAD_DB;
    if constexpr (GG) {
      // Stage this region's stored Z (same layout) with 16-B DMA loads:
      // load j covers rows 8j..8j+7; lane: row 8j + L/8, slot L%8.
      const i32x4 rZ = make_rsrc(a.Zin + cbase, a.c_bytes);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = j * 8 + (lane >> 3);
        const int c = quad_slot(row, lane & 7);
        const int gr = qm0 + row, gc = qn0 + c * 8;
        const uint32_t voff = (gr < a.M && gc < a.N)
                                  ? static_cast<uint32_t>((static_cast<int64_t>(gr) * a.ldc + gc) * 2)
                                  : OOB;
        buffer_load_lds16(rZ, lds + wave * QBYTES + j * 1024, voff);
      }
      wait_vmcnt<0>();
    }

    // EPI_GELU_GRAD_DB: this lane's column sums, over the wave's 128 rows,
    // of the values as stored (bf16-rounded); entry 4q + e of cs[j] is
    // column qn0 + 32j + 8q + 4·half + e
    float cs[FB][16];
    if constexpr (EPI == EPI_GELU_GRAD_DB) {
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) cs[j][e] = 0.f;
    }
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      // accumulators -> bf16 -> staging region, one 32×32 block at a time
#pragma unroll
      for (int i = 0; i < FA; ++i) {
        i32x2 zr[FB][4];
        // EPI_STORE_ROWSTATS: this lane's row statistics over its 32 of the
        // wave's 64 columns, of the values as stored (bf16-rounded)
        float rmx = -INFINITY, rsm = 0.f;
        if constexpr (BIAS) {
#pragma unroll
          for (int j = 0; j < FB; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              asm volatile("ds_read_b64 %0, %1" : "=v"(zr[j][q]) : "v"(bbase + (j * 32 + q * 8 + half * 4) * 2));
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(zr[0][0]), "+v"(zr[0][1]), "+v"(zr[0][2]), "+v"(zr[0][3]), "+v"(zr[1][0]),
                         "+v"(zr[1][1]), "+v"(zr[1][2]), "+v"(zr[1][3])::"memory");
        }
        if constexpr (GG) {
#pragma unroll
          for (int j = 0; j < FB; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              asm volatile("ds_read_b64 %0, %1"
                           : "=v"(zr[j][q])
                           : "v"(quad_addr(qbase, i * 32 + row_l, j * 4 + q, half)));
          // the Z registers are operands of the wait: no use moves above it
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(zr[0][0]), "+v"(zr[0][1]), "+v"(zr[0][2]), "+v"(zr[0][3]), "+v"(zr[1][0]),
                         "+v"(zr[1][1]), "+v"(zr[1][2]), "+v"(zr[1][3])::"memory");
        }
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          // The block's 16 accumulators are read in program order (volatile
          // asm keeps them behind the previous block's LDS writes), so only
          // one block is live in VGPRs and its 16 independent GeLU chains
          // interleave to cover the VALU latency.
          float v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[i][j][e]));
          if constexpr (BIAS) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bf16x4 bq = __builtin_bit_cast(bf16x4, zr[j][q]);
#pragma unroll
              for (int e = 0; e < 4; ++e) v[4 * q + e] += bf2f(bq[e]);
            }
          }
          if constexpr (ZY) {
            if (pass == 1) {
#pragma unroll
              for (int e = 0; e < 16; ++e) v[e] = gelu_fast(v[e]);
            }
          } else if constexpr (GG) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bf16x4 z = __builtin_bit_cast(bf16x4, zr[j][q]);
#pragma unroll
              for (int e = 0; e < 4; ++e) v[4 * q + e] *= gelu_grad_fast(bf2f(z[e]));
            }
          }
          i32x2 pk[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) pk[q] = pack4_bf16(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          if constexpr (EPI == EPI_GELU_GRAD_DB) {
            // rows past M and columns past N hold zeros (zero-filled operands)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t w = static_cast<uint32_t>(pk[q][e >> 1]);
                cs[j][4 * q + e] += __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
              }
          }
          if constexpr (EPI == EPI_STORE_ROWSTATS) {
            // value 4q + e is column qn0 + 32j + 8q + 4·half + e; columns past N
            // take no part
            float x[16];
            float bm = -INFINITY;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t w = static_cast<uint32_t>(pk[q][e >> 1]);
                const float y = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                x[4 * q + e] = qn0 + 32 * j + 8 * q + 4 * half + e < a.N ? y : -INFINITY;
                bm = fmaxf(bm, x[4 * q + e]);
              }
            if (bm > rmx) {
              rsm *= __expf(rmx - bm);
              rmx = bm;
            }
            if (rmx != -INFINITY) {
#pragma unroll
              for (int e = 0; e < 16; ++e) rsm += __expf(x[e] - rmx);
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            asm volatile("ds_write_b64 %0, %1" ::"v"(quad_addr(qbase, i * 32 + row_l, j * 4 + q, half)),
                         "v"(pk[q])
                         : "memory");
        }
        if constexpr (EPI == EPI_STORE_ROWSTATS) {
          // the row's two halves sit in lanes L and L+32: merge, and one of
          // them writes the pair of the wave's 64-column group
          const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmx), __float_as_uint(rmx), false, false);
          const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(rsm), __float_as_uint(rsm), false, false);
          const float m0 = __uint_as_float(pm[0]), m1 = __uint_as_float(pm[1]);
          const float s0 = __uint_as_float(ps[0]), s1 = __uint_as_float(ps[1]);
          const float mm = fmaxf(m0, m1);
          const float ss = mm == -INFINITY ? 0.f : s0 * __expf(m0 - mm) + s1 * __expf(m1 - mm);
          const int row = qm0 + i * 32 + row_l;
          const int ng = (a.N + 63) >> 6;
          if (half == 0 && row < a.M && qn0 < a.N) {
            float* r = a.rstats + (static_cast<int64_t>(batch) * a.M + row) * ng * 2 + (qn0 >> 6) * 2;
            r[0] = mm;
            r[1] = ss;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // staging region -> global: 8 rows × 128 B per wave-wide 16-B access
      bf16* C = static_cast<bf16*>(pass == 0 ? a.C : a.C2) + cbase;
#pragma unroll
      for (int it0 = 0; it0 < 16; it0 += 8) {
        i32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = (it0 + u) * 8 + (lane >> 3);
          const uint32_t ad = qbase + row * QROW + (quad_slot(row, lane & 7) << 4);
          asm volatile("ds_read_b128 %0, %1" : "=v"(v[u]) : "v"(ad) : "memory");
        }
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                       "+v"(v[7])::"memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = (it0 + u) * 8 + (lane >> 3);
          const int gr = qm0 + row, gc = qn0 + (lane & 7) * 8;
          // whole 128-B lines, not re-read by this launch: streamed past the L2
          // (leaves it to the A and B panels)
          if (gr < a.M && gc < a.N)
            __builtin_nontemporal_store(v[u], reinterpret_cast<i32x4*>(C + static_cast<int64_t>(gr) * a.ldc + gc));
        }
      }
    }
    if constexpr (EPI == EPI_GELU_GRAD_DB) {
      // sum over the 32 rows of each half (lanes of one half hold one row
      // each), in a fixed butterfly order; lane 0 / 32 then holds the wave's
      // 128-row column sums of its half's columns
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = cs[j][e];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o, 64);
          cs[j][e] = x;
        }
      const int64_t nchunk = (a.M + 127) / 128;
      const int64_t chunk = qm0 / 128;
      if (row_l == 0 && chunk < nchunk) {
        float* out = a.colsum + (static_cast<int64_t>(batch) * nchunk + chunk) * a.N;
#pragma unroll
        for (int j = 0; j < FB; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = qn0 + 32 * j + 8 * q + 4 * half;
            if (col < a.N) {
              f32x4 w;
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = cs[j][4 * q + e];
              *reinterpret_cast<f32x4*>(out + col) = w;
            }
          }
      }
    }
  }
  }  // TN == 256
}

// ---------------------------------------------------------------------------
// Epilogue of the 256×192 and 256×128 tiles.  Each wave stages its 64×(TN/2)
// bf16 region in LDS (rows of 256 B: chunk c of 8 columns of row r at 16-B
// slot c ^ (r % 16); 16 KiB per wave), then all 8 waves store the whole
// 256×TN tile together: a tile row is 2·TN bytes (three or two 128-B lines),
// and each wave-wide 16-B store writes 8 whole lines.  Z and Y (the GeLU
// epilogues) take one pass each, with a workgroup barrier before each pass's
// stores and after them.  Accumulator v of block (i, j) of lane L: row
// wm·64 + 32i + L%32, columns wn·TN/2 + 32j + 8·(v/4) + 4·(L/32) + v%4
// (wm = wave / 2, wn = wave % 2).
constexpr int NARROW_QROW = 256, NARROW_QBYTES = 64 * NARROW_QROW;
static_assert(NWAVE * NARROW_QBYTES + NWAVE * 256 <= LDS_BYTES, "narrow-tile epilogue staging exceeds the LDS");

__device__ __forceinline__ uint32_t narrow_addr(uint32_t qbase, int row, int chunk) {
  return qbase + row * NARROW_QROW + ((chunk ^ (row & 15)) << 4);
}

// fp32 results of the 256×128 tile (the K-split's partial planes): each
// wave stages its 64×64 fp32 region (rows of 256 B, 16-B chunk c of 4 floats
// at slot c ^ (row % 16)), then the 8 waves store the 256×128 tile together,
// 8 whole 128-B lines per wave-wide store.
__device__ void epilogue_narrow_f32(const KArgs& a, f32x16 (&acc)[2][2], int batch, int m0, int n0,
                                   TPMLP_LDS char* lds) {
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_l = lane & 31, half = lane >> 5;
  const uint32_t qbase = lds_base + wave * NARROW_QBYTES;
  block_barrier();  // every wave is done with the main-loop stages
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = i * 32 + row_l;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[i][j][e]));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = v[4 * q + e];
        // columns 32j + 8q + 4·half .. +3: chunk 8j + 2q + half of the region row
        asm volatile("ds_write_b128 %0, %1" ::"v"(narrow_addr(qbase, row, 8 * j + 2 * q + half)), "v"(w)
                     : "memory");
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  block_barrier();  // every region is staged
  // the tile: 256 rows × 32 chunks of 4 floats, 16 per thread
  float* C = static_cast<float*>(a.C) + static_cast<int64_t>(batch) * a.sC;
#pragma unroll
  for (int it0 = 0; it0 < 16; it0 += 8) {
    f32x4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int flat = (it0 + u) * NTHR + static_cast<int>(threadIdx.x);
      const int R = flat >> 5, c = flat & 31;
      const int rw = (R >> 6) * 2 + (c >> 4), rr = R & 63, cc = c & 15;
      asm volatile("ds_read_b128 %0, %1" : "=v"(w[u]) : "v"(narrow_addr(lds_base + rw * NARROW_QBYTES, rr, cc))
                   : "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      asm volatile("" : "+v"(w[u]));
      const int flat = (it0 + u) * NTHR + static_cast<int>(threadIdx.x);
      const int R = flat >> 5, c = flat & 31;
      const int gr = m0 + R, gc = n0 + c * 4;
      if (gr < a.M && gc < a.N) *reinterpret_cast<f32x4*>(C + static_cast<int64_t>(gr) * a.ldc + gc) = w[u];
    }
  }
}

template <int EPI, int TN>
__device__ void epilogue_narrow(const KArgs& a, f32x16 (&acc)[2][TN / 64], int batch, int m0, int n0,
                                TPMLP_LDS char* lds) {
  static_assert(TN == 192 || TN == 128, "narrow tile width");
  static_assert(EPI == EPI_STORE || EPI == EPI_GELU_ZY || EPI == EPI_BIAS_GELU_ZY || EPI == EPI_BIAS_STORE ||
                    EPI == EPI_GELU_GRAD || (EPI == EPI_STORE_F32 && TN == 128),
                "epilogue not available for the narrow tiles");
  if constexpr (EPI == EPI_STORE_F32) {
    epilogue_narrow_f32(a, acc, batch, m0, n0, lds);
    return;
  } else {
  constexpr int NJ = TN / 64;        // 32-column blocks per wave
  constexpr int CH = TN / 16;        // 16-B chunks per region row
  constexpr int TCH = TN / 8;        // 16-B chunks per tile row
  constexpr int ITER = 256 * TCH / NTHR;  // chunks stored per thread
  constexpr bool ZY = EPI == EPI_GELU_ZY || EPI == EPI_BIAS_GELU_ZY;
  constexpr bool BIAS = EPI == EPI_BIAS_GELU_ZY || EPI == EPI_BIAS_STORE;
  constexpr bool GG = EPI == EPI_GELU_GRAD;
  constexpr int PASSES = ZY ? 2 : 1;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int row_l = lane & 31, half = lane >> 5;
  const uint32_t qbase = lds_base + wave * NARROW_QBYTES;
  const int64_t cbase = static_cast<int64_t>(batch) * a.sC;
  const int qm0 = m0 + wm * 64, qn0 = n0 + wn * (TN / 2);
  block_barrier();  // every wave is done with the main-loop stages

  // column bias: the wave's TN/2 values, staged past the staging regions
  const uint32_t bbase = lds_base + NWAVE * NARROW_QBYTES + wave * 256;
  if constexpr (BIAS) {
    if (lane < TN / 8) {
      const int col = qn0 + lane * 4;
      const bf16* bias = a.bias + static_cast<int64_t>(batch) * a.sBias;
      const i32x2 b = col < a.N ? *reinterpret_cast<const i32x2*>(bias + col) : i32x2{0, 0};
      asm volatile("ds_write_b64 %0, %1" ::"v"(bbase + lane * 8), "v"(b) : "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if constexpr (GG) {
    // the region's stored Z in the staging layout: load j fills rows
    // 4j..4j+3 (1 KiB); lane: row 4j + L/16, slot L%16, chunk slot ^ (row % 16)
    const i32x4 rZ = make_rsrc(a.Zin + cbase, a.c_bytes);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = j * 4 + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      const int gr = qm0 + row, gc = qn0 + c * 8;
      const uint32_t voff = (c < CH && gr < a.M && gc < a.N)
                                ? static_cast<uint32_t>((static_cast<int64_t>(gr) * a.ldc + gc) * 2)
                                : OOB;
      buffer_load_lds16(rZ, lds + wave * NARROW_QBYTES + j * 1024, voff);
    }
    wait_vmcnt<0>();
  }

#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = i * 32 + row_l;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        i32x2 zr[4];
        if constexpr (BIAS) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            asm volatile("ds_read_b64 %0, %1" : "=v"(zr[q]) : "v"(bbase + (j * 32 + q * 8 + half * 4) * 2));
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(zr[0]), "+v"(zr[1]), "+v"(zr[2]), "+v"(zr[3])::"memory");
        }
        if constexpr (GG) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            asm volatile("ds_read_b64 %0, %1" : "=v"(zr[q]) : "v"(narrow_addr(qbase, row, j * 4 + q) + half * 8));
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(zr[0]), "+v"(zr[1]), "+v"(zr[2]), "+v"(zr[3])::"memory");
        }
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[i][j][e]));
        if constexpr (BIAS) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bf16x4 bq = __builtin_bit_cast(bf16x4, zr[q]);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] += bf2f(bq[e]);
          }
        }
        if constexpr (ZY) {
          if (pass == 1) {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = gelu_fast(v[e]);
          }
        } else if constexpr (GG) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bf16x4 z = __builtin_bit_cast(bf16x4, zr[q]);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] *= gelu_grad_fast(bf2f(z[e]));
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x2 pk = pack4_bf16(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          asm volatile("ds_write_b64 %0, %1" ::"v"(narrow_addr(qbase, row, j * 4 + q) + half * 8), "v"(pk)
                       : "memory");
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();  // every region of this pass is staged
    // the tile: 256 rows × TCH chunks, ITER per thread; thread t, round it:
    // chunk it·512 + t in row-major order
    bf16* C = static_cast<bf16*>(pass == 0 ? a.C : a.C2) + cbase;
#pragma unroll
    for (int it0 = 0; it0 < ITER; it0 += ITER / 2) {
      i32x4 w[ITER / 2];
#pragma unroll
      for (int u = 0; u < ITER / 2; ++u) {
        const int flat = (it0 + u) * NTHR + static_cast<int>(threadIdx.x);
        const int R = flat / TCH, c = flat - R * TCH;
        const int rw = (R >> 6) * 2 + (c >= CH ? 1 : 0), rr = R & 63, cc = c >= CH ? c - CH : c;
        const uint32_t ad = narrow_addr(lds_base + rw * NARROW_QBYTES, rr, cc);
        asm volatile("ds_read_b128 %0, %1" : "=v"(w[u]) : "v"(ad) : "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < ITER / 2; ++u) {
        asm volatile("" : "+v"(w[u]));
        const int flat = (it0 + u) * NTHR + static_cast<int>(threadIdx.x);
        const int R = flat / TCH, c = flat - R * TCH;
        const int gr = m0 + R, gc = n0 + c * 8;
        if (gr < a.M && gc < a.N)
          __builtin_nontemporal_store(w[u], reinterpret_cast<i32x4*>(C + static_cast<int64_t>(gr) * a.ldc + gc));
      }
    }
    if (pass + 1 < PASSES) block_barrier();  // the staging regions are read before the next pass writes them
  }
  }  // not fp32
}

// The launch: problems 0 and 1 are of kind (AO0, BO0, EPI0), problem 2 of
// kind (AO1, BO1, EPI1).
// A tile of a K-split problem: its slice s (the slowest index of the tile
// order, so one slice's tiles run together) becomes a problem of its own over
// k in [s·kchunk, min(K, (s+1)·kchunk)): the operands' base pointers and
// buffer ranges move to the slice's first k (the K-edge test zero-fills the
// rest) and the fp32 partial goes to the slice's plane.
template <int AO, int BO>
__device__ __forceinline__ void select_slice(KArgs& a, int& tile) {
  if (a.ksplit <= 1) return;
  const int per_slice = a.tiles_m * a.tiles_n * a.batch;
  const int slice = tile / per_slice;
  tile -= slice * per_slice;
  const int k0 = slice * a.kchunk;
  const int rest = a.K - k0;
  a.K = rest < a.kchunk ? (rest > 0 ? rest : 0) : a.kchunk;
  const int64_t offA = AO == KMAJ ? k0 : static_cast<int64_t>(k0) * a.lda;
  const int64_t offB = BO == KMAJ ? k0 : static_cast<int64_t>(k0) * a.ldb;
  a.A += offA;
  a.B += offB;
  a.a_bytes = a.a_bytes > offA * 2 ? a.a_bytes - static_cast<uint32_t>(offA * 2) : 0u;
  a.b_bytes = a.b_bytes > offB * 2 ? a.b_bytes - static_cast<uint32_t>(offB * 2) : 0u;
  a.C = static_cast<float*>(a.C) + slice * a.sSlice;
}

// Restrict problem a to k in [k0, k0 + len): the operands' base pointers and
// buffer ranges move to k0 (the K-edge test zero-fills past the new K).
template <int AO, int BO>
__device__ __forceinline__ void shift_k(KArgs& a, int k0, int len) {
  const int64_t offA = AO == KMAJ ? k0 : static_cast<int64_t>(k0) * a.lda;
  const int64_t offB = BO == KMAJ ? k0 : static_cast<int64_t>(k0) * a.ldb;
  a.A += offA;
  a.B += offB;
  a.a_bytes = a.a_bytes > offA * 2 ? a.a_bytes - static_cast<uint32_t>(offA * 2) : 0u;
  a.b_bytes = a.b_bytes > offB * 2 ? a.b_bytes - static_cast<uint32_t>(offB * 2) : 0u;
  a.K = len;
}

// Tail item c of problem a (a.sk_L > 0): piece j of tail tile u, an fp32
// partial tile in slot c.
template <int AO, int BO>
__device__ __forceinline__ void sk_item(const KArgs& a, int c, TPMLP_LDS char* lds) {
  const int j = c / a.sk_T, u = c - j * a.sk_T;
  const int kb = j * a.sk_L;
  if (j >= a.sk_q || kb >= a.sk_KS) return;  // the whole workgroup: c is uniform
  const int ke = kb + a.sk_L < a.sk_KS ? kb + a.sk_L : a.sk_KS;
  int batch, tm, tn;
  tile_coords(u + a.sk_first, a, batch, tm, tn);
  KArgs b = a;
  const int k0 = kb * BK;
  const int rest = a.K - k0;
  const int len = (ke - kb) * BK < rest ? (ke - kb) * BK : rest;
  shift_k<AO, BO>(b, k0, len);
  // the slot holds the tile at row stride 256; the epilogue adds
  // (batch·sC + row·ldc + col) to C, so C is moved back by the tile origin
  float* slot = a.sk_ws + static_cast<int64_t>(c) * (BM * BN);
  b.C = slot - (static_cast<int64_t>(tm) * BM * BN + static_cast<int64_t>(tn) * BN);
  b.ldc = BN;
  b.sC = 0;
  gemm_tile<AO, BO, EPI_STORE_F32>(b, u + a.sk_first, lds);
}

template <int AO0, int BO0, int EPI0, int AO1, int BO1, int EPI1, int TN = BN>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(KGroup g) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  TPMLP_LDS char* lds = (TPMLP_LDS char*)(smem);
  int prob, tile;
  map_workgroup(g.split, g.t0, blockIdx.x, prob, tile);
  if constexpr (TN != BN) {
    // narrow tiles: launches of one kind (fp32: a K-split's slices)
    static_assert(AO0 == AO1 && BO0 == BO1 && EPI0 == EPI1, "one kind per narrow-tile launch");
    KArgs a = g.p[prob];
    if constexpr (EPI0 == EPI_STORE_F32) select_slice<AO0, BO0>(a, tile);
    gemm_tile<AO0, BO0, EPI0, TN>(a, tile, lds);
  } else if constexpr (AO0 == AO1 && BO0 == BO1 && EPI0 == EPI1) {
    KArgs a = g.p[prob];  // one copy: wide scalar loads at the problem's offset
    if constexpr (EPI0 == EPI_STORE_F32) select_slice<AO0, BO0>(a, tile);
    gemm_tile<AO0, BO0, EPI0>(a, tile, lds);
  } else {
    KArgs a = g.p[prob];
    if (prob == 2) {
      if constexpr (EPI1 == EPI_STORE_F32) {
        if (a.sk_L > 0) {
          sk_item<AO1, BO1>(a, tile, lds);
          return;
        }
        select_slice<AO1, BO1>(a, tile);
      }
      gemm_tile<AO1, BO1, EPI1>(a, tile, lds);
    } else {
      if constexpr (EPI0 == EPI_STORE_F32) select_slice<AO0, BO0>(a, tile);
      gemm_tile<AO0, BO0, EPI0>(a, tile, lds);
    }
  }
}

// ------------------------------------------------------------------ split-K fix-up
// out = epilogue(Σ_{s<S} part[s]) for one problem that ran K-split: the
// slices' fp32 partial tiles are added in slice order (a fixed order, so the
// result is bit-reproducible) and the problem's own epilogue is applied with
// the same fp32 arithmetic as the unsplit kernel's.  A thread owns 8
// consecutive columns of one row (N % 8 == 0).
struct FixArgs {
  const float* part;  // [S][batch][M][N]
  int S, batch, M, N;
  int64_t sSlice;     // batch·M·N
  void* C;
  void* C2;
  const bf16* Zin;
  const bf16* bias;
  int64_t sBias, ldc, sC;
};

constexpr int FIX_THREADS = 256;

// The epilogue of a fixed-up sum x of 8 consecutive columns at element offset
// o of the output (bias offset ob): the same fp32 arithmetic as the GEMM's own
// epilogue.
template <int EPI>
__device__ __forceinline__ void fix_store(float (&x)[8], int64_t o, int64_t ob, void* C, void* C2, const bf16* Zin,
                                          const bf16* bias) {
  if constexpr (EPI == EPI_BIAS_GELU_ZY || EPI == EPI_BIAS_STORE) {
    const bf16x8 bb = *reinterpret_cast<const bf16x8*>(bias + ob);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += bf2f(bb[e]);
  }
  if constexpr (EPI == EPI_STORE_F32) {
    f32x4 lo, hi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo[q] = x[q];
      hi[q] = x[4 + q];
    }
    float* c = static_cast<float*>(C) + o;
    reinterpret_cast<f32x4*>(c)[0] = lo;
    reinterpret_cast<f32x4*>(c)[1] = hi;
  } else {
    bf16x8 r;
    if constexpr (EPI == EPI_GELU_GRAD) {
      const bf16x8 z = *reinterpret_cast<const bf16x8*>(Zin + o);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = f2bf(x[e] * gelu_grad_fast(bf2f(z[e])));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = f2bf(x[e]);
    }
    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(C) + o) = r;
    if constexpr (EPI == EPI_GELU_ZY || EPI == EPI_BIAS_GELU_ZY) {
      bf16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = f2bf(gelu_fast(x[e]));
      *reinterpret_cast<bf16x8*>(static_cast<bf16*>(C2) + o) = y;
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(FIX_THREADS) void splitk_fixup_kernel(FixArgs f) {
  const int64_t nvec = static_cast<int64_t>(f.batch) * f.M * (f.N / 8);
  const int64_t step = static_cast<int64_t>(gridDim.x) * FIX_THREADS;
  const int64_t per_b = static_cast<int64_t>(f.M) * (f.N / 8);
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * FIX_THREADS + threadIdx.x; v < nvec; v += step) {
    const int64_t b = v / per_b;
    const int64_t rem = v - b * per_b;
    const int64_t row = rem / (f.N / 8);
    const int64_t col = (rem - row * (f.N / 8)) * 8;
    const float* src = f.part + (b * f.M + row) * f.N + col;
    float x[8];
    {
      const f32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
      const f32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src) + 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[q] = lo[q];
        x[4 + q] = hi[q];
      }
    }
    for (int sl = 1; sl < f.S; ++sl) {
      const f32x4* q4 = reinterpret_cast<const f32x4*>(src + sl * f.sSlice);
      const f32x4 lo = __builtin_nontemporal_load(q4), hi = __builtin_nontemporal_load(q4 + 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[q] += lo[q];
        x[4 + q] += hi[q];
      }
    }
    fix_store<EPI>(x, b * f.sC + row * f.ldc + col, b * f.sBias + col, f.C, f.C2, f.Zin, f.bias);
  }
}

// Tail fix-up: out = epilogue(Σ_j piece j) for the tail tiles of problem a,
// the pieces added in K order, so the result is bit-reproducible.  32 blocks
// per tile; a thread owns 8 consecutive columns of one row.
template <int EPI>
__global__ __launch_bounds__(FIX_THREADS) void sk_fixup_kernel(KArgs a) {
  const int u = static_cast<int>(blockIdx.x >> 5);
  const int v = static_cast<int>(blockIdx.x & 31) * FIX_THREADS + static_cast<int>(threadIdx.x);
  const int r = v >> 5, cc = (v & 31) * 8;
  int batch, tm, tn;
  tile_coords(u + a.sk_first, a, batch, tm, tn);
  const int64_t row = static_cast<int64_t>(tm) * BM + r, col = static_cast<int64_t>(tn) * BN + cc;
  if (row >= a.M || col >= a.N) return;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.f;
  for (int j = 0; j < a.sk_q; ++j) {
    const int64_t slot = static_cast<int64_t>(j) * a.sk_T + u;
    const f32x4* q4 = reinterpret_cast<const f32x4*>(a.sk_ws + slot * (BM * BN) + r * BN + cc);
    const f32x4 lo = __builtin_nontemporal_load(q4), hi = __builtin_nontemporal_load(q4 + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] += lo[q];
      x[4 + q] += hi[q];
    }
  }
  fix_store<EPI>(x, static_cast<int64_t>(batch) * a.sC + row * a.ldc + col,
                 static_cast<int64_t>(batch) * a.sBias + col, a.C, a.C2, a.Zin, a.bias);
}

template <int AO0, int BO0, int EPI0, int AO1, int BO1, int EPI1, int TN = BN>
hipError_t launch_t(const KGroup& g, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_bf16_kernel<AO0, BO0, EPI0, AO1, BO1, EPI1, TN>), dim3(g.t0 + g.t1 + g.t2), dim3(NTHR), 0,
                     stream, g);
  return hipGetLastError();
}

uint32_t extent_bytes(int order, int rows, int K, int64_t ld) {
  // bytes spanned by a rows×K operand of the given storage order
  if (rows <= 0 || K <= 0) return 0;
  int64_t elems = order == KMAJ ? (static_cast<int64_t>(rows) - 1) * ld + K
                                : (static_cast<int64_t>(K) - 1) * ld + rows;
  return static_cast<uint32_t>(elems * 2);
}


KArgs kargs(const GemmProblem& p, int a_order, int b_order, int tn = BN) {
  KArgs k{};  // every field zero unless set below (no K split, no stream-K items)
  k.A = static_cast<const bf16*>(p.A);
  k.B = static_cast<const bf16*>(p.B);
  k.C = p.C;
  k.C2 = p.C2;
  k.Zin = static_cast<const bf16*>(p.Zin);
  k.bias = static_cast<const bf16*>(p.bias);
  k.sBias = p.sBias;
  k.rstats = p.rstats;
  k.colsum = p.colsum;
  k.M = p.M;
  k.N = p.N;
  k.K = p.K;
  k.tiles_m = (p.M + BM - 1) / BM;
  k.tiles_n = (p.N + tn - 1) / tn;
  k.batch = p.batch;
  k.lda = p.lda;
  k.ldb = p.ldb;
  k.ldc = p.ldc;
  k.sA = p.sA;
  k.sB = p.sB;
  k.sC = p.sC;
  k.a_bytes = extent_bytes(a_order, p.M, p.K, p.lda);
  k.b_bytes = extent_bytes(b_order, p.N, p.K, p.ldb);
  k.c_bytes = static_cast<uint32_t>(((static_cast<int64_t>(p.M) - 1) * p.ldc + p.N) * 2);
  k.ksplit = 1;
  k.kchunk = p.K;
  k.sSlice = 0;
  return k;
}

bool empty(const GemmProblem& p) { return p.M <= 0 || p.N <= 0 || p.batch <= 0; }

int64_t tiles_of(const GemmProblem& p, int tn = BN) {
  return empty(p) ? 0 : static_cast<int64_t>((p.M + BM - 1) / BM) * ((p.N + tn - 1) / tn) * p.batch;
}

// ---------------------------------------------------------------- split-K plan
// A launch whose tiles cannot fill the 256 CUs, or whose longest tiles leave
// most of the machine idle at the end, runs some problems K-split: slice s of
// S computes its fp32 partial tile over a contiguous range of K, and a fix-up
// kernel adds the S partials in slice order and applies the problem's
// epilogue.  The choice minimises a cost model in units of one K step (64) of
// a tile on a loaded machine: the launch takes about max(longest tile,
// total tile work / 256 CUs), each tile also pays a fixed prologue/epilogue,
// and a split pays the S fp32 partial planes twice (the GEMM's epilogue
// writes them, the fix-up kernel reads them) and the fix-up's launch.  The
// choice depends only on the shapes, so a call is bit-reproducible.
// Measured on the single-shard layer (n = 2048, d = 1024, m = 4096): a
// 16-step tile takes 31 µs alone on the GPU, about 1.5 µs per step plus
// ≈ 6 µs; P = Y·B split in 4 takes 32 + 7 µs (fix-up), split in 8 36 + 13 µs
// (256 tiles writing 64 MB of fp32 partials at once), unsplit ≈ 100 µs.
constexpr double kTileFixedSteps = 4.0;     // a tile's prologue + epilogue
constexpr double kFixBytesPerStep = 6.4e6;  // partial-plane traffic per step time (≈ 4 TB/s × 1.6 µs)
constexpr double kFixLaunchSteps = 2.0;
constexpr int kCUs = 256;
constexpr int kMinStepsPerSlice = 8;

struct SplitPlan {
  int s[3];
  size_t off[3];  // byte offset of each split problem's partial planes in the workspace
  size_t bytes;
  // K-split tail (sk_slot >= 0): that problem's first sk_first tiles run as
  // whole tiles, the sk_T after them as sk_q pieces of sk_L K steps each
  int sk_slot, sk_L, sk_T, sk_first, sk_KS, sk_q;
  size_t sk_off;
};

bool splittable(const GemmKind& k) { return k.epi != EPI_STORE_ROWSTATS && k.epi != EPI_GELU_GRAD_DB; }

std::atomic<int> g_tile_policy{TILE_AUTO};

// Output bytes per element of a kind's epilogue (the fix-up's writes and reads
// beyond the partials).
double out_bytes(const GemmKind& k) {
  switch (k.epi) {
    case EPI_GELU_ZY:
    case EPI_BIAS_GELU_ZY:
    case EPI_GELU_GRAD: return 4.0;
    case EPI_STORE_F32: return 4.0;
    default: return 2.0;
  }
}

// K-split tail for a launch of one problem whose tiles fill r ≥ 1 whole
// rounds of the kCUs CUs and then at most half of one more: the last Tt =
// T − r·kCUs tiles are each split into q = min(⌊kCUs/Tt⌋, KS) pieces of L =
// ⌈KS/q⌉ K steps, all Tt·q ≤ kCUs pieces running as one extra round, and a
// fix-up adds each tile's pieces in order and applies the epilogue.  The
// pieces of one index j cover the same K range in every tail tile, so tiles
// that share an operand panel read it together (a stream-K split into equal
// ranges of the tail's whole step sequence cut tiles at different K and
// made the panels of a launch with a large B operand, the GPT-1T-shaped
// shard's Z = X·A_i, be read once per tile: slower than no split).  Cost, in
// K steps of a tile: r whole rounds, one piece round, and the partial planes
// written and read plus the outputs at kFixBytesPerStep.
void plan_stream_k(SplitPlan& pl, const GemmProblem* const (&pr)[3], const GemmKind* const (&kd)[3], int policy) {
  pl.sk_slot = -1;
  if (policy == TILE_256 || policy == TILE_192 || policy == TILE_128) return;
  int live = -1, nlive = 0;
  for (int i = 0; i < 3; ++i)
    if (pr[i] != nullptr && !empty(*pr[i])) {
      live = i;
      ++nlive;
    }
  if (nlive != 1 || pl.s[live] > 1) return;
  const GemmProblem& p = *pr[live];
  const GemmKind& k = *kd[live];
  if (!splittable(k) || k.epi == EPI_STORE_F32 || p.N % 8 != 0) return;
  const int64_t T = tiles_of(p);
  const int KS = (p.K + BK - 1) / BK;
  const int64_t r = T / kCUs, Tt = T - r * kCUs;
  if (r < 1 || Tt == 0 || KS < 2) return;
  int64_t q = kCUs / Tt;
  if (q > KS) q = KS;
  if (q < 2) return;
  const int64_t L = (KS + q - 1) / q;
  q = (KS + L - 1) / L;  // pieces that are not empty
  const double now = static_cast<double>(r + 1) * (KS + kTileFixedSteps);
  const double bytes = static_cast<double>(Tt) * q * BM * BN * 4.0 * 2.0 + static_cast<double>(Tt) * BM * BN * out_bytes(k);
  const double sk = static_cast<double>(r) * (KS + kTileFixedSteps) + L + kTileFixedSteps +
                    bytes / kFixBytesPerStep + kFixLaunchSteps;
  if (policy != TILE_STREAMK && !(sk < 0.95 * now)) return;
  pl.sk_slot = live;
  pl.sk_L = static_cast<int>(L);
  pl.sk_T = static_cast<int>(Tt);
  pl.sk_q = static_cast<int>(q);
  pl.sk_first = static_cast<int>(r * kCUs);
  pl.sk_KS = KS;
  pl.sk_off = pl.bytes;
  pl.bytes += static_cast<size_t>(Tt * q) * BM * BN * 4;
}

// problems: up to three (null = absent); kinds: theirs
SplitPlan plan_split(const GemmProblem* const (&pr)[3], const GemmKind* const (&kd)[3]) {
  SplitPlan best{{1, 1, 1}, {0, 0, 0}, 0, -1, 0, 0, 0, 0, 0, 0};
  double T[3], KS[3], MN[3];
  bool can[3];
  for (int i = 0; i < 3; ++i) {
    const bool live = pr[i] != nullptr && !empty(*pr[i]);
    T[i] = live ? static_cast<double>(tiles_of(*pr[i])) : 0.0;
    KS[i] = live ? static_cast<double>((pr[i]->K + BK - 1) / BK) : 0.0;
    MN[i] = live ? static_cast<double>(pr[i]->batch) * pr[i]->M * pr[i]->N : 0.0;
    can[i] = live && splittable(*kd[i]) && pr[i]->N % 8 == 0;
  }
  auto cost = [&](const int (&s)[3]) {
    double longest = 0.0, work = 0.0, fix = 0.0;
    for (int i = 0; i < 3; ++i) {
      if (T[i] == 0.0) continue;
      const double c = static_cast<double>((static_cast<int64_t>(KS[i]) + s[i] - 1) / s[i]) + kTileFixedSteps;
      longest = c > longest ? c : longest;
      work += T[i] * s[i] * c;
      if (s[i] > 1) fix += 2.0 * s[i] * MN[i] * 4.0 / kFixBytesPerStep + kFixLaunchSteps;
    }
    const double spread = work / kCUs;
    return (longest > spread ? longest : spread) + fix;
  };
  int s[3] = {1, 1, 1};
  double bc = cost(s);
  static const int kS[5] = {1, 2, 4, 8, 16};
  for (int a = 0; a < 5; ++a)
    for (int b = 0; b < 5; ++b)
      for (int c = 0; c < 5; ++c) {
        const int cand[3] = {kS[a], kS[b], kS[c]};
        bool ok = true;
        for (int i = 0; i < 3; ++i)
          if (cand[i] > 1 && (!can[i] || KS[i] < kMinStepsPerSlice * cand[i])) ok = false;
        // the two long problems share one kind: split alike unless that kind
        // already is the fp32 store a split runs as
        if (T[0] > 0.0 && T[1] > 0.0 && kd[0]->epi != EPI_STORE_F32 && cand[0] != cand[1]) ok = false;
        if (!ok) continue;
        const double cc = cost(cand);
        if (cc < bc * 0.97) {  // a split must win clearly
          bc = cc;
          for (int i = 0; i < 3; ++i) s[i] = cand[i];
        }
      }
  size_t off = 0;
  for (int i = 0; i < 3; ++i) {
    best.s[i] = s[i];
    best.off[i] = off;
    if (s[i] > 1) off += (static_cast<size_t>(s[i]) * static_cast<size_t>(MN[i]) * 4 + 255) / 256 * 256;
  }
  best.bytes = off;
  plan_stream_k(best, pr, kd, g_tile_policy.load(std::memory_order_relaxed));
  return best;
}

hipError_t fixup(const GemmProblem& p, int epi, const float* part, int S, hipStream_t stream) {
  FixArgs f;
  f.part = part;
  f.S = S;
  f.batch = p.batch;
  f.M = p.M;
  f.N = p.N;
  f.sSlice = static_cast<int64_t>(p.batch) * p.M * p.N;
  f.C = p.C;
  f.C2 = p.C2;
  f.Zin = static_cast<const bf16*>(p.Zin);
  f.bias = static_cast<const bf16*>(p.bias);
  f.sBias = p.sBias;
  f.ldc = p.ldc;
  f.sC = p.sC;
  const int64_t nvec = static_cast<int64_t>(p.batch) * p.M * (p.N / 8);
  int64_t blocks = (nvec + FIX_THREADS - 1) / FIX_THREADS;
  if (blocks > 8192) blocks = 8192;
  const dim3 grid(static_cast<unsigned>(blocks)), block(FIX_THREADS);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(splitk_fixup_kernel<EPI_STORE>, grid, block, 0, stream, f); break;
    case EPI_STORE_F32: hipLaunchKernelGGL(splitk_fixup_kernel<EPI_STORE_F32>, grid, block, 0, stream, f); break;
    case EPI_GELU_ZY: hipLaunchKernelGGL(splitk_fixup_kernel<EPI_GELU_ZY>, grid, block, 0, stream, f); break;
    case EPI_GELU_GRAD: hipLaunchKernelGGL(splitk_fixup_kernel<EPI_GELU_GRAD>, grid, block, 0, stream, f); break;
    case EPI_BIAS_GELU_ZY:
      hipLaunchKernelGGL(splitk_fixup_kernel<EPI_BIAS_GELU_ZY>, grid, block, 0, stream, f);
      break;
    case EPI_BIAS_STORE: hipLaunchKernelGGL(splitk_fixup_kernel<EPI_BIAS_STORE>, grid, block, 0, stream, f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- tile width
// A launch of one kind that runs unsplit may take the 256×192 tile instead of
// 256×256 when that fills the 256 CUs in fewer rounds of tiles: 8192×1536 is
// 192 tiles of 256×256 (three quarters of the CUs for one round) or 256 of
// 256×192 (all of them); 8192×3072 is 384 (two rounds, the second half empty)
// or 512 (two full ones).  Cost of a round, in K steps of a 256×256 tile: the
// steps plus the fixed prologue/epilogue.  A 256×192 step does 3/4 of the
// MFMA work but moves 7/8 of the operand bytes, and the K loop is bound by
// that stream: measured on one shard of the 8.3B-shaped layer, 72.8 against
// 81.0 µs (Z = X·A_i, 48 steps, one round each) and 72.3 against 80.7 µs
// (P = Y·B_i, 24 steps, two rounds each), i.e. 0.9 of a step per step.  Only
// shapes decide, so a call is reproducible.
constexpr double k192StepFrac = 0.9, k192FixedSteps = 3.5;
// 256×128 tiles: half the MFMA work and 3/4 of the operand bytes per step.
// Measured on the single-shard layer's Z = X·A and dgrad-1 (2048×4096
// outputs, 16 K steps; 256 tiles of 256×128 against 176 of 256×192, one round
// each): 23.4 and 25.0 µs against 27.3 and 27.4 µs, i.e. about 0.85 of the
// 256×192 round, which the constants reproduce.
constexpr double k128StepFrac = 0.8, k128FixedSteps = 3.0;

bool n192_kind(const GemmKind& k) {
  if (k.a_order != KMAJ) return false;
  if (k.b_order == MNMAJ)
    return k.epi == EPI_STORE || k.epi == EPI_GELU_ZY || k.epi == EPI_BIAS_GELU_ZY || k.epi == EPI_BIAS_STORE;
  return k.epi == EPI_STORE || k.epi == EPI_GELU_GRAD;
}

// A launch of 256×TN tiles (TN = 192 or 128) of one kind.
template <int TN>
hipError_t launch_narrow(const KGroup& g, const GemmKind& k, hipStream_t stream) {
  auto is = [&](int ao, int bo, int epi) { return k.a_order == ao && k.b_order == bo && k.epi == epi; };
  if (is(KMAJ, MNMAJ, EPI_GELU_ZY)) return launch_t<KMAJ, MNMAJ, EPI_GELU_ZY, KMAJ, MNMAJ, EPI_GELU_ZY, TN>(g, stream);
  if (is(KMAJ, MNMAJ, EPI_BIAS_GELU_ZY))
    return launch_t<KMAJ, MNMAJ, EPI_BIAS_GELU_ZY, KMAJ, MNMAJ, EPI_BIAS_GELU_ZY, TN>(g, stream);
  if (is(KMAJ, MNMAJ, EPI_STORE)) return launch_t<KMAJ, MNMAJ, EPI_STORE, KMAJ, MNMAJ, EPI_STORE, TN>(g, stream);
  if (is(KMAJ, MNMAJ, EPI_BIAS_STORE))
    return launch_t<KMAJ, MNMAJ, EPI_BIAS_STORE, KMAJ, MNMAJ, EPI_BIAS_STORE, TN>(g, stream);
  if (is(KMAJ, KMAJ, EPI_GELU_GRAD)) return launch_t<KMAJ, KMAJ, EPI_GELU_GRAD, KMAJ, KMAJ, EPI_GELU_GRAD, TN>(g, stream);
  if (is(KMAJ, KMAJ, EPI_STORE)) return launch_t<KMAJ, KMAJ, EPI_STORE, KMAJ, KMAJ, EPI_STORE, TN>(g, stream);
  if constexpr (TN == 128) {
    if (is(KMAJ, MNMAJ, EPI_STORE_F32))
      return launch_t<KMAJ, MNMAJ, EPI_STORE_F32, KMAJ, MNMAJ, EPI_STORE_F32, TN>(g, stream);
    if (is(KMAJ, KMAJ, EPI_STORE_F32))
      return launch_t<KMAJ, KMAJ, EPI_STORE_F32, KMAJ, KMAJ, EPI_STORE_F32, TN>(g, stream);
  }
  return hipErrorInvalidValue;
}

// A launch planned with a K-split tail: the first sk_first tiles as whole
// tiles (problem 0, the problem's own epilogue), the sk_T·sk_q tail pieces as
// problem 2 (fp32 partials), then the fix-up over the sk_T tail tiles.
hipError_t launch_stream_k(const GemmProblem& p, const GemmKind& k, const SplitPlan& pl, char* wsb,
                           hipStream_t stream) {
  KGroup g;
  const KArgs a = kargs(p, k.a_order, k.b_order);
  KArgs b = a;
  b.sk_L = pl.sk_L;
  b.sk_T = pl.sk_T;
  b.sk_first = pl.sk_first;
  b.sk_KS = pl.sk_KS;
  b.sk_q = pl.sk_q;
  b.sk_ws = reinterpret_cast<float*>(wsb + pl.sk_off);
  g.p[0] = a;
  g.p[1] = a;
  g.p[2] = b;
  g.t0 = pl.sk_first;
  g.t1 = 0;
  g.t2 = pl.sk_T * pl.sk_q;
  g.split = make_split(g.t0, g.t1, g.t2);
  auto is = [&](int ao, int bo, int epi) { return k.a_order == ao && k.b_order == bo && k.epi == epi; };
  hipError_t e = hipErrorInvalidValue;
  if (is(KMAJ, MNMAJ, EPI_GELU_ZY))
    e = launch_t<KMAJ, MNMAJ, EPI_GELU_ZY, KMAJ, MNMAJ, EPI_STORE_F32>(g, stream);
  else if (is(KMAJ, MNMAJ, EPI_BIAS_GELU_ZY))
    e = launch_t<KMAJ, MNMAJ, EPI_BIAS_GELU_ZY, KMAJ, MNMAJ, EPI_STORE_F32>(g, stream);
  else if (is(KMAJ, MNMAJ, EPI_STORE))
    e = launch_t<KMAJ, MNMAJ, EPI_STORE, KMAJ, MNMAJ, EPI_STORE_F32>(g, stream);
  else if (is(KMAJ, MNMAJ, EPI_BIAS_STORE))
    e = launch_t<KMAJ, MNMAJ, EPI_BIAS_STORE, KMAJ, MNMAJ, EPI_STORE_F32>(g, stream);
  else if (is(KMAJ, KMAJ, EPI_GELU_GRAD))
    e = launch_t<KMAJ, KMAJ, EPI_GELU_GRAD, KMAJ, KMAJ, EPI_STORE_F32>(g, stream);
  else if (is(KMAJ, KMAJ, EPI_STORE))
    e = launch_t<KMAJ, KMAJ, EPI_STORE, KMAJ, KMAJ, EPI_STORE_F32>(g, stream);
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(pl.sk_T) * 32), block(FIX_THREADS);
  switch (k.epi) {
    case EPI_STORE: hipLaunchKernelGGL(sk_fixup_kernel<EPI_STORE>, grid, block, 0, stream, b); break;
    case EPI_GELU_ZY: hipLaunchKernelGGL(sk_fixup_kernel<EPI_GELU_ZY>, grid, block, 0, stream, b); break;
    case EPI_GELU_GRAD: hipLaunchKernelGGL(sk_fixup_kernel<EPI_GELU_GRAD>, grid, block, 0, stream, b); break;
    case EPI_BIAS_GELU_ZY: hipLaunchKernelGGL(sk_fixup_kernel<EPI_BIAS_GELU_ZY>, grid, block, 0, stream, b); break;
    case EPI_BIAS_STORE: hipLaunchKernelGGL(sk_fixup_kernel<EPI_BIAS_STORE>, grid, block, 0, stream, b); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

void set_gemm_tile_policy(int policy) { g_tile_policy.store(policy, std::memory_order_relaxed); }
int gemm_tile_policy() { return g_tile_policy.load(std::memory_order_relaxed); }

size_t gemm_bf16_split_bytes(const GemmProblem* longp, int nlong, const GemmKind& long_kind,
                             const GemmProblem* shortp, const GemmKind& short_kind) {
  const GemmProblem* pr[3] = {nlong > 0 ? &longp[0] : nullptr, nlong > 1 ? &longp[1] : nullptr, shortp};
  const GemmKind* kd[3] = {&long_kind, &long_kind, &short_kind};
  return plan_split(pr, kd).bytes;
}

hipError_t launch_gemm_bf16_group(const GemmProblem* longp, int nlong, const GemmKind& long_kind,
                                  const GemmProblem* shortp, const GemmKind& short_kind, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (nlong < 0 || nlong > 2 || (nlong > 0 && longp == nullptr)) return hipErrorInvalidValue;
  // the split plan over the three problem slots (long 0, long 1, short)
  const GemmProblem* slot[3] = {nlong > 0 ? &longp[0] : nullptr, nlong > 1 ? &longp[1] : nullptr, shortp};
  const GemmKind* kslot[3] = {&long_kind, &long_kind, &short_kind};
  SplitPlan plan = plan_split(slot, kslot);
  if (ws == nullptr || ws_bytes < plan.bytes) plan = SplitPlan{{1, 1, 1}, {0, 0, 0}, 0, -1, 0, 0, 0, 0, 0, 0};
  char* wsb = static_cast<char*>(ws);
  if (plan.sk_slot >= 0) return launch_stream_k(*slot[plan.sk_slot], *kslot[plan.sk_slot], plan, wsb, stream);

  // a K-split problem runs as an fp32 store of its slices' partials
  GemmProblem sp[3];
  GemmKind sk[3];
  for (int i = 0; i < 3; ++i) {
    if (slot[i] == nullptr) continue;
    sp[i] = *slot[i];
    sk[i] = *kslot[i];
    if (plan.s[i] > 1) {
      sp[i].C = wsb + plan.off[i];
      sp[i].C2 = nullptr;
      sp[i].ldc = sp[i].N;
      sp[i].sC = static_cast<int64_t>(sp[i].M) * sp[i].N;
      sk[i].epi = EPI_STORE_F32;
    }
  }
  // the long group has one kind: split or not, its problems must agree
  if (nlong == 2 && plan.s[0] > 1 && plan.s[1] > 1 && sk[0].epi != sk[1].epi) return hipErrorInvalidValue;
  if (nlong == 2 && (plan.s[0] > 1) != (plan.s[1] > 1) && long_kind.epi != EPI_STORE_F32)
    return hipErrorInvalidValue;

  const GemmProblem* lp[2];
  int li[2];
  int nl = 0;
  for (int i = 0; i < nlong; ++i)
    if (!empty(sp[i])) {
      lp[nl] = &sp[i];
      li[nl++] = i;
    }
  const bool has_short = shortp != nullptr && !empty(sp[2]);
  const GemmKind lk = nl > 0 ? sk[li[0]] : long_kind;
  const GemmKind shk = has_short ? sk[2] : short_kind;
  // with no long-group problem the launch is of the short kind alone, and
  // vice versa
  const GemmKind& k0 = nl > 0 ? lk : shk;
  const GemmKind& k1 = has_short ? shk : lk;
  auto is = [](const GemmKind& x, int ao, int bo, int epi) {
    return x.a_order == ao && x.b_order == bo && x.epi == epi;
  };
  const bool same = is(k1, k0.a_order, k0.b_order, k0.epi);
  int tn = BN;
  const int policy = g_tile_policy.load(std::memory_order_relaxed);
  if (policy != TILE_256 && same && n192_kind(k0) && plan.s[0] <= 1 && plan.s[1] <= 1 &&
      plan.s[2] <= 1) {
    int64_t T256 = 0, T192 = 0, T128 = 0;
    int ks = 0;
    for (int i = 0; i < 3; ++i) {
      if (slot[i] == nullptr || empty(sp[i]) || (i == 2 && !has_short) || (i < 2 && i >= nlong)) continue;
      T256 += tiles_of(sp[i]);
      T192 += tiles_of(sp[i], 192);
      T128 += tiles_of(sp[i], 128);
      const int k = (sp[i].K + BK - 1) / BK;
      ks = k > ks ? k : ks;
    }
    auto rounds = [](int64_t T) { return static_cast<double>((T + kCUs - 1) / kCUs); };
    const double c256 = rounds(T256) * (ks + kTileFixedSteps);
    const double c192 = rounds(T192) * (k192StepFrac * ks + k192FixedSteps);
    const double c128 = rounds(T128) * (k128StepFrac * ks + k128FixedSteps);
    if (policy == TILE_192) tn = 192;
    else if (policy == TILE_128) tn = 128;
    else if (c192 < 0.95 * c256 && c192 <= c128) tn = 192;
    else if (c128 < 0.95 * c256) tn = 128;
  } else if (policy != TILE_256 && policy != TILE_192 && same && k0.epi == EPI_STORE_F32 && k0.a_order == KMAJ &&
             nl + (has_short ? 1 : 0) == 1) {
    // one K-split problem (its slices are fp32 stores): 256×128 tiles when
    // its slices leave the CUs partly idle (the single-shard layer's P = Y·B:
    // 32 tiles × 4 slices of 256×256, 64 × 4 of 256×128)
    const int i = nl > 0 ? li[0] : 2;
    const int S = plan.s[i];
    if (S > 1) {
      const int steps = ((sp[i].K + BK - 1) / BK + S - 1) / S;
      auto rounds = [](int64_t T) { return static_cast<double>((T + kCUs - 1) / kCUs); };
      const double c256 = rounds(tiles_of(sp[i]) * S) * (steps + kTileFixedSteps);
      const double c128 = rounds(tiles_of(sp[i], 128) * S) * (k128StepFrac * steps + k128FixedSteps);
      if (policy == TILE_128 || c128 < 0.95 * c256) tn = 128;
    }
  }
  const int64_t t0 = nl > 0 ? tiles_of(*lp[0], tn) * plan.s[li[0]] : 0;
  const int64_t t1 = nl > 1 ? tiles_of(*lp[1], tn) * plan.s[li[1]] : 0;
  const int64_t t2 = has_short ? tiles_of(sp[2], tn) * plan.s[2] : 0;
  if (t0 + t1 + t2 == 0) return hipSuccess;
  if (t0 + t1 + t2 > 0x7fffffff) return hipErrorInvalidValue;
  KGroup g;
  auto mk = [&](const GemmProblem& q, int i, const GemmKind& k) {
    KArgs a = kargs(q, k.a_order, k.b_order, tn);
    if (plan.s[i] > 1) {
      const int ks = (q.K + BK - 1) / BK;
      a.ksplit = plan.s[i];
      a.kchunk = (ks + plan.s[i] - 1) / plan.s[i] * BK;
      a.sSlice = static_cast<int64_t>(q.batch) * q.M * q.N;
    }
    return a;
  };
  g.p[0] = nl > 0 ? mk(*lp[0], li[0], lk) : KArgs{};
  g.p[1] = nl > 1 ? mk(*lp[1], li[1], lk) : g.p[0];
  g.p[2] = has_short ? mk(sp[2], 2, shk) : g.p[0];
  g.t0 = static_cast<int>(t0);
  g.t1 = static_cast<int>(t1);
  g.t2 = static_cast<int>(t2);
  // longest tiles first: the short problem's before the long group's when its
  // tiles take more K steps (e.g. dgrad-2, K = m_i, against weight gradients
  // with K = n at few tokens)
  auto steps = [](const KArgs& a) { return a.ksplit > 1 ? a.kchunk / BK : (a.K + BK - 1) / BK; };
  const bool short_first = nl > 0 && has_short && steps(g.p[2]) > steps(g.p[0]);
  g.split = make_split(g.t0, g.t1, g.t2, short_first);
  hipError_t e = hipErrorInvalidValue;
  if (tn == 192)
    e = launch_narrow<192>(g, k0, stream);
  else if (tn == 128)
    e = launch_narrow<128>(g, k0, stream);  // (its fp32 kind: a K-split's slices, fixed up below)
  else if (same && is(k0, KMAJ, MNMAJ, EPI_GELU_ZY))
    e = launch_t<KMAJ, MNMAJ, EPI_GELU_ZY, KMAJ, MNMAJ, EPI_GELU_ZY>(g, stream);
  else if (same && is(k0, KMAJ, MNMAJ, EPI_BIAS_GELU_ZY))
    e = launch_t<KMAJ, MNMAJ, EPI_BIAS_GELU_ZY, KMAJ, MNMAJ, EPI_BIAS_GELU_ZY>(g, stream);
  else if (same && is(k0, KMAJ, MNMAJ, EPI_STORE))
    e = launch_t<KMAJ, MNMAJ, EPI_STORE, KMAJ, MNMAJ, EPI_STORE>(g, stream);
  else if (same && is(k0, KMAJ, MNMAJ, EPI_BIAS_STORE))
    e = launch_t<KMAJ, MNMAJ, EPI_BIAS_STORE, KMAJ, MNMAJ, EPI_BIAS_STORE>(g, stream);
  else if (same && is(k0, KMAJ, MNMAJ, EPI_STORE_F32))
    e = launch_t<KMAJ, MNMAJ, EPI_STORE_F32, KMAJ, MNMAJ, EPI_STORE_F32>(g, stream);
  else if (same && is(k0, KMAJ, KMAJ, EPI_GELU_GRAD))
    e = launch_t<KMAJ, KMAJ, EPI_GELU_GRAD, KMAJ, KMAJ, EPI_GELU_GRAD>(g, stream);
  else if (same && is(k0, KMAJ, KMAJ, EPI_GELU_GRAD_DB))
    e = launch_t<KMAJ, KMAJ, EPI_GELU_GRAD_DB, KMAJ, KMAJ, EPI_GELU_GRAD_DB>(g, stream);
  else if (same && is(k0, KMAJ, KMAJ, EPI_STORE))
    e = launch_t<KMAJ, KMAJ, EPI_STORE, KMAJ, KMAJ, EPI_STORE>(g, stream);
  else if (same && is(k0, KMAJ, KMAJ, EPI_STORE_ROWSTATS))
    e = launch_t<KMAJ, KMAJ, EPI_STORE_ROWSTATS, KMAJ, KMAJ, EPI_STORE_ROWSTATS>(g, stream);
  else if (same && is(k0, KMAJ, KMAJ, EPI_STORE_F32))
    e = launch_t<KMAJ, KMAJ, EPI_STORE_F32, KMAJ, KMAJ, EPI_STORE_F32>(g, stream);
  else if (same && is(k0, MNMAJ, MNMAJ, EPI_STORE_F32))
    e = launch_t<MNMAJ, MNMAJ, EPI_STORE_F32, MNMAJ, MNMAJ, EPI_STORE_F32>(g, stream);
  // the backward's last launch: both weight gradients, then dgrad-2 (as
  // itself, or as its K-split fp32 partials)
  else if (is(k0, MNMAJ, MNMAJ, EPI_STORE_F32) && is(k1, KMAJ, KMAJ, EPI_STORE))
    e = launch_t<MNMAJ, MNMAJ, EPI_STORE_F32, KMAJ, KMAJ, EPI_STORE>(g, stream);
  else if (is(k0, MNMAJ, MNMAJ, EPI_STORE_F32) && is(k1, KMAJ, KMAJ, EPI_STORE_F32))
    e = launch_t<MNMAJ, MNMAJ, EPI_STORE_F32, KMAJ, KMAJ, EPI_STORE_F32>(g, stream);
  if (e != hipSuccess) return e;
  // the fix-ups, in slot order
  for (int i = 0; i < 3; ++i) {
    if (slot[i] == nullptr || plan.s[i] <= 1 || empty(sp[i])) continue;
    e = fixup(*slot[i], kslot[i]->epi, reinterpret_cast<const float*>(wsb + plan.off[i]), plan.s[i], stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_bf16(const GemmProblem& p, int a_order, int b_order, int epi, hipStream_t stream) {
  const GemmKind k{a_order, b_order, epi};
  return launch_gemm_bf16_group(&p, 1, k, nullptr, k, nullptr, 0, stream);
}

hipError_t launch_gemm_bf16_ws(const GemmProblem& p, int a_order, int b_order, int epi, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  const GemmKind k{a_order, b_order, epi};
  return launch_gemm_bf16_group(&p, 1, k, nullptr, k, ws, ws_bytes, stream);
}

}  // namespace tpmlp
