// bf16 MFMA GEMM for gfx950: the grouped expert GEMMs and the dense latent projections.
//
// What it computes ("Как устроен Olmo-core 3: обучение больших MoE-моделей"):
//   * section "Вычисления экспертов и точность": tokens grouped by expert run through each
//     expert's MLP with a grouped matrix multiply over int32 row offsets; the grouped experts
//     return bf16;
//   * section "SwiGLU с квантизацией": the first matrix's output splits into halves, up then
//     gate, and act = up * gate * sigmoid(gate) in fp32;
//   * section "Латентная проекция экспертов": the dense down-projection d_model -> latent_dim
//     and up-projection latent_dim -> d_model (dense mode: one group, M = tokens).
// All operands are "NT": token rows A (M, Kd) and weight rows B (N, Kd), Kd contiguous, fp32
// accumulation.
//
// Design for CDNA4:
//   * v_mfma_f32_32x32x16_bf16. The weight rows feed the MFMA's first operand and the token
//     rows its second, so each lane ends with 4 consecutive output columns of one token row
//     (8 bytes of packed bf16) and the SwiGLU pairs up/gate in registers.
//   * Tile = (WM*TM*32 token rows) x (WN*TN*32 weight rows) x 64 k, WM x WN wavefronts. The
//     large variant is 256 x 256 with 8 wavefronts (2 x 4) of 128 token rows x 64 weight rows
//     (8 MFMA accumulators of 16 floats each). LDS holds two stages of both tiles (128 KiB);
//     16-byte chunks are XOR-swizzled by row pair so fragment reads are free of bank conflicts.
//   * The A loader gathers token rows through the permutation (row = perm[p] / k), so the
//     permuted copy of the tokens is never materialised; the GEMM2 epilogue scatters rows to
//     assignment order, so the combine reads each token's k rows contiguously.
//   * Persistent grid (one workgroup per CU slot). Workgroup i runs on XCD i % 8; the linear
//     tile sequence goes in groups of 4 M-tiles x all N-tiles and is cut into 8 contiguous
//     chunks, one per XCD, so the tiles an XCD runs together share A and B panels in that
//     XCD's L2. Tile lists dominated by experts of 16 or more M-tiles are instead dealt to the
//     XCDs tile by tile, so the XCDs run neighbouring groups of one expert together and share
//     panels through the last-level cache as well. Small tiles use only as many workgroups of
//     an XCD as finish its chunk in the same number of rounds, so no round runs part-empty.
//   * Operands reach LDS by DMA (16 bytes per lane, no register round trip); each 64-k stage
//     is one whole 128-byte line per staged row. Every operand loads with buffer_load ... lds:
//     row-major operands and contraction-major weights through one descriptor per operand,
//     the k-stage step a scalar offset; the weight gradients' operands through a descriptor per
//     stage whose range ends at the group's last row, so rows past it read as zeros. Measured
//     on the same box, that streams faster than global_load_lds (a 32768 x 4096 x 4096 dense
//     product 1191 -> 1248 TFLOP/s), and the operand loads need no per-lane 64-bit addresses.
//     (The MXFP8 scale rows keep global_load_lds: descriptors measured within noise there.)
//   * Staggered load issue (large tiles, weight-gradient tiles): of the two wavefronts sharing a
//     SIMD, one issues its share of the next stage's loads before its first fragment reads, the
//     other after its first k16 step, so the pair does not stall together on a full address
//     queue.
//   * Epilogue through LDS: the accumulators leave the MFMA layout as 8-byte pieces of 32
//     different rows, so stored directly every instruction writes 32 partial lines. They are
//     staged in the free ring slot instead and stored as whole rows (full 128-byte lines per
//     instruction). Large bf16 tiles issue the next tile's first stage as the epilogue starts
//     (its list entry and row indices were fetched during the current tile), other shapes
//     during the last staging round.
//   * Experts with no tokens have no M-tile and their weights are never read.
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;
constexpr int kGroupM = 4;

template <int WM_, int WN_, int TM_, int TN_, int BK_, int NSTAGE_, int WG_PER_CU_, int PLANES_ = 1, int EB_ = 2,
          int SCG_ = 1>
struct Shape {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  // Bytes per operand element: 2 = bf16; 1 = MXFP8 (E4M3 codes with one E8M0 scale byte per
  // 32 elements along k, multiplied on v_mfma_scale_f32_32x32x64_f8f6f4).
  static constexpr int EB = EB_;
  static constexpr bool MX = EB == 1;
  // Weight planes summed into one product (3 for the fp32 router: its weights split exactly
  // into three bf16 planes); each stage then stages PLANES x BN weight rows.
  static constexpr int PLANES = PLANES_;
  static constexpr int BK = BK_;                // k per pipeline stage
  static constexpr int ROWB = BK * EB;          // bytes per staged row
  static constexpr int CHUNKS = ROWB / 16;      // 16-byte chunks per staged row
  static constexpr int ROWS_PER_BANKLINE = 256 / ROWB;  // rows sharing the 64 LDS banks
  static constexpr int kRowsPerDma = 1024 / ROWB;       // rows one wave-wide 16-byte DMA load fills
  static constexpr int NSTAGE = NSTAGE_;        // LDS ring depth; loads run NSTAGE-1 stages ahead
  static constexpr int WG_PER_CU = WG_PER_CU_;  // resident workgroups per CU (persistent grid)
  static constexpr int NW = WM * WN;            // wavefronts
  static constexpr int NT = NW * kWave;         // threads
  static constexpr int BM = WM * TM * 32;       // token rows
  static constexpr int BN = WN * TN * 32;       // weight rows
  static constexpr int BROWS = PLANES * BN;     // staged weight rows
  static constexpr int NI = (BM + BROWS) / kRowsPerDma;  // DMA loads per stage
  static constexpr int NQ = (NI + NW - 1) / NW;        // per wavefront (upper bound)
  static constexpr int NQMIN = NI / NW;                // per wavefront (lower bound)
  static constexpr int DATA = (BM + BROWS) * ROWB;  // operand bytes per stage
  // MXFP8 scales: 4 bytes per staged row and k-stage (k-stage 128 = four blocks of 32), one
  // DMA load per 64 rows. SCG = 1: each stage's scale bytes follow its operands (4 bytes per
  // lane). SCG = 4: the scales of four consecutive k-stages travel together (16 bytes per lane,
  // issued with every fourth stage, a quarter of the line requests) into a two-group area
  // after the ring: group g serves stages 4g..4g+3 from half g % 2.
  static constexpr int SCG = MX ? SCG_ : 0;
  static constexpr int SCB = MX ? BK / 32 : 0;
  static constexpr int NSC = MX ? (BM + BROWS) / 64 : 0;
  static constexpr int STAGE = DATA + (SCG == 1 ? (BM + BROWS) * SCB : 0);
  static constexpr int SCHALF = SCG == 4 ? (BM + BROWS) * 16 : 0;  // bytes per scale group
  static constexpr int LDS = NSTAGE * STAGE + 2 * SCHALF;
  static_assert(!MX || (BK == 128 && PLANES == 1 && BM % 64 == 0 && BN % 64 == 0 && NSC <= NW),
                "MXFP8 stages: 128-element k-stages, 64-row scale loads, one per wavefront");
  static_assert(!MX || SCG == 1 || SCG == 4, "scale groups of one or four k-stages");
  static_assert(BM % kRowsPerDma == 0 && BN % kRowsPerDma == 0, "whole DMA loads per tile");
  static_assert(BK % 16 == 0 && CHUNKS >= 2 && CHUNKS <= 8, "stage depth");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "vmcnt bookkeeping covers 2..4 stages");
  static_assert(LDS * WG_PER_CU <= 160 * 1024, "LDS budget");
};

// The load path (texture addresser / L1, 128-byte lines) is the scarce resource of these GEMMs,
// more than the matrix pipes: every staged row is one whole 128-byte line (k-stage 64), and
// tiles are as large as LDS allows so each line feeds as many MFMAs as possible.
// 256 x 256 tile, 8 wavefronts (2 x 4) of 128 token rows x 64 weight rows; 2 stages x 64 KiB.
using ShapeLarge = Shape<2, 4, 4, 2, 64, 2, 1>;
// 64 x 256 tile, 4 wavefronts (1 x 4) of 64 x 64: few rows per expert (decode-shaped loads);
// 2 stages x 40 KiB, two workgroups per CU.
using ShapeSmall = Shape<1, 4, 2, 2, 64, 2, 2>;
// MXFP8 expert GEMMs: the large tile with 128-element k-stages (one 128-byte line of E4M3 codes
// per row) plus the rows' scale bytes; 2 stages x 66 KiB.
using ShapeLargeMX = Shape<2, 4, 4, 2, 128, 2, 1, 1, 1>;
// The same with the scales of four k-stages per load (k a multiple of 512): 2 stages x 64 KiB
// plus 2 x 8 KiB of scale groups.
using ShapeLargeMXG = Shape<2, 4, 4, 2, 128, 2, 1, 1, 1, 4>;
// Router logits: 256 tokens x 128 experts x 3 weight planes, 8 wavefronts (2 x 4) of 128 x 32;
// 2 stages x 80 KiB (the whole LDS).
using ShapeRouter = Shape<2, 4, 4, 1, 64, 2, 1, 3>;

// LDS is 64 banks of 4 bytes and a 16-byte access serves 16 lanes per pass. A staged row covers
// 1/ROWS_PER_BANKLINE of the banks; chunk c of row r lives in slot c ^ ((r / ROWS_PER_BANKLINE)
// & (CHUNKS - 1)), so the 16 consecutive rows of one fragment read (same chunk) hit 16 distinct
// 16-byte bank groups. DMA writes are linear in the lane index: conflict-free by construction.
template <class S>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * S::ROWB + ((chunk ^ ((row / S::ROWS_PER_BANKLINE) & (S::CHUNKS - 1))) << 4);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// 8- and 16-byte LDS writes through inline asm, for the epilogue's staging: the compiler's
// wait-count insertion does not count them as LDS accesses, so it does not hold them until
// DMA loads in flight into the other ring slot have landed (it cannot always prove the two
// LDS arrays apart). The epilogue waits for them itself (lgkmcnt) before the barrier that
// publishes them; "memory" keeps them in order with the other memory operations.
typedef uint32_t u32x2s __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_store_b64(void* p, uint32_t lo, uint32_t hi) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(p)));
  const u32x2s d = {lo, hi};
  asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(d) : "memory");
}
__device__ __forceinline__ void lds_store_b128(void* p, float x, float y, float z, float w) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(p)));
  const u32x4s d = {__float_as_uint(x), __float_as_uint(y), __float_as_uint(z), __float_as_uint(w)};
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(d) : "memory");
}

// Instruction-scheduling directives for one pipeline stage: step 0's LDS reads first, then in
// each k16 step pair MFMAs with the next step's LDS reads and with this stage's share of the
// global->LDS loads, so neither the LDS round trip nor the address unit stalls the matrix pipe.
// (Masks: 0x008 MFMA, 0x010 VMEM, 0x100 DS read.)
template <int KK, int KSTEPS, int KREADS, int KMFMA, int KLOADS, int LEFT>
__device__ __forceinline__ void sched_stage_step() {
  if constexpr (KK < KSTEPS) {
    constexpr int reads = (KK + 1 < KSTEPS) ? KREADS : 0;
    constexpr int per = (KLOADS + KSTEPS - 1) / KSTEPS;
    constexpr int loads = LEFT < per ? LEFT : per;
    constexpr int r1 = reads < KMFMA ? reads : KMFMA;
    constexpr int l1 = loads < (KMFMA - r1) ? loads : (KMFMA - r1);
#pragma unroll
    for (int q = 0; q < r1; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (reads > r1) __builtin_amdgcn_sched_group_barrier(0x100, reads - r1, 0);
#pragma unroll
    for (int q = 0; q < l1; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
    if constexpr (loads > l1) __builtin_amdgcn_sched_group_barrier(0x010, loads - l1, 0);
    if constexpr (KMFMA - r1 - l1 > 0) __builtin_amdgcn_sched_group_barrier(0x008, KMFMA - r1 - l1, 0);
    sched_stage_step<KK + 1, KSTEPS, KREADS, KMFMA, KLOADS, LEFT - loads>();
  }
}

// One MXFP8 MFMA: a and b hold 32 E4M3 codes of a row per lane (bytes 0-15 from the first
// 32-element block of the 64-k step, bytes 16-31 from the second: each lane supplies its half
// of both blocks), sa / sb the E8M0 scale of block (lane / 32) of the lane's row (lane % 32)
// in byte 0.
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, static_cast<int>(sa), 0,
                                                         static_cast<int>(sb));
}

// Contraction-major operands (the backward's W^T, dY^T and act^T products): a staged row is one
// contraction index with the tile's 256 columns (512 bytes, 32 chunks of 16 bytes); chunk c of
// row r lives in slot c ^ ((r & 3) << 2), so the four rows one transposing read touches per
// half-wavefront land in four different quarters of the banks.
constexpr int kTrRowBytes = 512;
__device__ __forceinline__ int tr_addr(int row, int col) {
  return row * kTrRowBytes + ((((col >> 3) ^ ((row & 3) << 2))) << 4) + ((col & 7) << 1);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// MFMA fragment (8 consecutive contraction indices of one column) from a contraction-major
// tile: ds_read_b64_tr_b16 gives lane i of each 16-lane group element (i % 4) of the 8 bytes
// addressed by lane 4 * j + i / 4 of the group, for j = 0..3. Each lane therefore addresses
// row (i / 4) and columns 4 * (i % 4) .. +3 of a 4 x 16 block, and receives the four rows of
// column i: two reads give the 8 contraction indices of the lane's column. Lanes 0-15 / 16-31
// take columns 0-15 / 16-31 of the 32-column sub-tile at contraction 0-7 of the k16 step, lanes
// 32-63 the same columns at contraction 8-15 (the MFMA operand layout).
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* tile, int col32, int kk, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int col = col32 + 16 * (g & 1) + 4 * (i & 3);
  const int row = 16 * kk + 8 * (g >> 1) + (i >> 2);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + tr_addr(row, col)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + tr_addr(row + 4, col)));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// The same directives with a stage's KLOADS global->LDS loads placed as one group: before step 0's
// LDS reads (AT < 0) or right after the MFMAs of k16 step AT.
template <int KK, int KSTEPS, int KREADS, int KMFMA, int KLOADS, int AT>
__device__ __forceinline__ void sched_stage_loads_at_step() {
  if constexpr (KK < KSTEPS) {
    constexpr int reads = (KK + 1 < KSTEPS) ? KREADS : 0;
    constexpr int r1 = reads < KMFMA ? reads : KMFMA;
#pragma unroll
    for (int q = 0; q < r1; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (reads > r1) __builtin_amdgcn_sched_group_barrier(0x100, reads - r1, 0);
    if constexpr (KMFMA - r1 > 0) __builtin_amdgcn_sched_group_barrier(0x008, KMFMA - r1, 0);
    if constexpr (KK == AT) __builtin_amdgcn_sched_group_barrier(0x010, KLOADS, 0);
    sched_stage_loads_at_step<KK + 1, KSTEPS, KREADS, KMFMA, KLOADS, AT>();
  }
}
template <int KSTEPS, int KREADS, int KMFMA, int KLOADS, int AT>
__device__ __forceinline__ void sched_stage_loads_at() {
  if constexpr (AT < 0) __builtin_amdgcn_sched_group_barrier(0x010, KLOADS, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, KREADS, 0);  // step-0 reads
  sched_stage_loads_at_step<0, KSTEPS, KREADS, KMFMA, KLOADS, AT>();
}

template <int KSTEPS, int KREADS, int KMFMA, int KLOADS>
__device__ __forceinline__ void sched_stage() {
  __builtin_amdgcn_sched_group_barrier(0x100, KREADS, 0);  // step-0 reads
  sched_stage_step<0, KSTEPS, KREADS, KMFMA, KLOADS, KLOADS>();
}

// MXFP8 scale groups (shapes with four k-stages of scales per load): their own LDS array;
// other shapes have none.
template <class S>
__device__ __forceinline__ unsigned char* scale_area() {
  if constexpr (S::SCHALF > 0) {
    __shared__ __attribute__((aligned(1024))) unsigned char a[2 * S::SCHALF];
    return a;
  } else {
    return nullptr;
  }
}

// The kernel's work, for one tile order (SP: spread, see below); the kernel after it picks one.
// lds0 / lds1: the two ring slots, separate LDS arrays, so the compiler can tell that DMA loads
// into one slot never touch another: it then does not hold the epilogue's staging in slot 1
// until the next tile's loads into slot 0 have landed.
template <class S, bool SWIGLU, bool GATHER, bool SCATTER, bool OUT_F32, bool OUT_MX, int TRANS, bool WGRAD,
          bool SWIGLU_BWD, bool H_OUT, bool SP>
__device__ __forceinline__ void gemm_bf16_body(const GemmCall& c, unsigned char* lds0, unsigned char* lds1) {
  static_assert(S::NSTAGE == 2, "the persistent loop runs a two-slot ring");
  constexpr bool TA = (TRANS & 1) != 0, TB = (TRANS & 2) != 0;
  static_assert(!(TA || TB) || (!S::MX && S::PLANES == 1 && S::BK == 64 && !SWIGLU && !OUT_F32 && !OUT_MX),
                "contraction-major operands: plain bf16 products");
  static_assert(!TA || S::BM * 2 == kTrRowBytes, "contraction-major A: 256-column tiles");
  static_assert(!TB || S::BN * 2 == kTrRowBytes, "contraction-major B: 256-column tiles");
  static_assert(!WGRAD || (TRANS == 3 && !GATHER && !SCATTER && !SWIGLU_BWD), "weight gradients: both operands contraction-major");
  static_assert(!SWIGLU_BWD || (!SWIGLU && !SCATTER && !OUT_F32 && !OUT_MX), "SwiGLU backward epilogue");
  static_assert(!H_OUT || (SWIGLU && !S::MX), "the pre-activation is stored by the bf16 SwiGLU GEMM");
  static_assert(!SWIGLU || S::TN % 2 == 0, "SwiGLU pairs up/gate sub-tiles inside a wavefront");
  static_assert(!SWIGLU || S::PLANES == 1, "planes are for plain products");
  using OutT = typename std::conditional<OUT_F32, float, uint16_t>::type;
  unsigned char* const ldssc = scale_area<S>();
  const int tid = threadIdx.x, lane = tid & 63;
  // wavefront coordinates are uniform per wavefront: keep them in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WN, wn = wave % S::WN;

  const int64_t cols_per_tile = SWIGLU ? S::BN / 2 : S::BN;
  const int64_t ntn = (c.N + cols_per_tile - 1) / cols_per_tile;
  // weight-gradient mode: every group has the same M-tiles (output rows of one group)
  const int64_t wg_mtiles = WGRAD ? (c.dense_M + S::BM - 1) / S::BM : 1;
  const int64_t total_m = WGRAD ? wg_mtiles * c.groups
                          : c.dense_M > 0 ? (c.dense_M + S::BM - 1) / S::BM
                                          : min(static_cast<int64_t>(*c.tiles.count),
                                                static_cast<int64_t>(c.tiles.cap));
  const int64_t total = total_m * ntn;
  const int xcd = blockIdx.x % kXcds;
  const int64_t chunk = (total + kXcds - 1) / kXcds;
  // Tiles go in groups of kGroupM M-tiles x all N-tiles (consecutive in the linear sequence),
  // and each XCD runs about 32 of them at a time: kGroupM M-tiles x 8 N-tiles, whose operand
  // panels share that XCD's L2. Spread order: XCD x takes tiles x, x + 8, x + 16, ... of the
  // sequence, so the eight XCDs run sixteen neighbouring M-tiles x all N-tiles at once, each
  // XCD still kGroupM M-tiles x half the N-tiles; every token panel is then shared by two XCDs
  // and every weight panel by four through the last-level cache. That pays where an expert
  // spans those sixteen M-tiles; with smaller experts an XCD's window would straddle several
  // experts, so there (and for dense products, where it measured no better) each XCD takes one
  // contiguous eighth of the sequence. The dispatch marks a main tile list (count[1]) when most
  // of its M-tiles belong to experts of at least kSpreadMinMTiles M-tiles; the kernel then runs
  // the SP copy of this body.
  // Small tiles stream weights from HBM, and a last round that only part of the workgroups
  // run leaves bandwidth unused: there only as many workgroups of the XCD take part as still
  // finish its share of the tiles in the same number of rounds, each taking the same number.
  // (Large tiles are bound by the matrix cores, where the slowest workgroup's tile count
  // decides either way.)
  int per_xcd = gridDim.x / kXcds;
  if constexpr (!WGRAD && S::WG_PER_CU > 1) {
    const int64_t rounds = (chunk + per_xcd - 1) / per_xcd;
    if (rounds > 0) per_xcd = static_cast<int>((chunk + rounds - 1) / rounds);
  }
  const unsigned char* Ab = static_cast<const unsigned char*>(c.A);
  // bytes from one k-stage to the next: along the row, or 64 rows down for a contraction-major
  // operand
  const uint32_t a_step = TA ? static_cast<uint32_t>(S::BK * c.lda * 2) : static_cast<uint32_t>(S::ROWB);
  const uint32_t b_step = TB ? static_cast<uint32_t>(S::BK * c.ldb * 2) : static_cast<uint32_t>(S::ROWB);
  OutT* Cbase = static_cast<OutT*>(c.C);

  // this lane's row inside a DMA load
  const int dma_row = lane / S::CHUNKS;

  // One output tile of the persistent sequence: where its rows and columns come from, the
  // source offsets of this wavefront's DMA loads, and the output rows of this lane.
  struct TileState {
    int64_t row0, nt;
    int rows;
    int nk;                    // k-stages of this tile
    int kcnt;                  // weight-gradient mode: contraction rows of the tile's group
    int64_t cofs;              // weight-gradient mode: output offset of the group (elements)
    const unsigned char* Abase;
    const unsigned char* Bexp;
    uint32_t src_off[S::NQ];  // byte offset of the source 16-byte chunk of load q (k-stage 0)
    const unsigned char* sc_base;  // MXFP8: scale array of this wavefront's 64 staged rows
    uint32_t sc_off;               // MXFP8: byte offset of this lane's row scales (k-stage 0)
  };
  // The load index inside a stage is uniform per wavefront, so is the operand it reads.
  auto load_is_a = [&](int q) { return wave + S::NW * q < S::BM / S::kRowsPerDma; };

  // What a tile's setup reads from memory, fetched one tile ahead (during the previous tile's
  // k-loop) so that the next tile's first loads can be issued as soon as its epilogue starts:
  // the tile's coordinates, its list entry, and the source row of each of this lane's
  // token-row loads (and, MXFP8, of its scale row).
  struct TileFetch {
    int64_t nt, row0, grp, kb;
    int rows, kcnt;
    int32_t src[S::NQ];  // token-row loads: source row of the A operand
    int32_t scsrc;       // MXFP8 scale loads of token rows: source row
  };

  // it: the tile's position in the linear sequence, or (weight-gradient mode) its index in the
  // heavy-first sequence handed out by the tile counter
  auto fetch = [&](int64_t it, TileFetch& f) {
    int64_t mt;
    if (WGRAD) {
      // groups in the given order (most rows first), each group's M-tiles x N-tiles in turn
      const int64_t per_group = wg_mtiles * ntn;
      const int64_t r = it / per_group, local = it - r * per_group;
      const int64_t g = c.group_order ? min(max(static_cast<int64_t>(c.group_order[r]), int64_t(0)),
                                            static_cast<int64_t>(c.groups) - 1)
                                      : r;
      mt = g * wg_mtiles + local / ntn;
      f.nt = local % ntn;
    } else {
      const int64_t lin = it;
      const int64_t gsz = kGroupM * ntn;
      const int64_t grp_i = lin / gsz, first_m = grp_i * kGroupM;
      const int64_t gm = min(static_cast<int64_t>(kGroupM), total_m - first_m);
      const int64_t local = lin - grp_i * gsz;
      mt = first_m + local % gm;
      f.nt = local / gm;
    }
    f.kcnt = 0;
    f.kb = 0;
    if (WGRAD) {
      f.grp = mt / wg_mtiles;
      f.row0 = (mt - f.grp * wg_mtiles) * S::BM;
      f.rows = static_cast<int>(min(static_cast<int64_t>(S::BM), c.dense_M - f.row0));
      const int64_t kb = min(max(static_cast<int64_t>(c.group_offsets[f.grp]), int64_t(0)), c.rows_bound);
      const int64_t ke = min(max(static_cast<int64_t>(c.group_offsets[f.grp + 1]), kb), c.rows_bound);
      f.kb = kb;
      f.kcnt = static_cast<int>(ke - kb);
    } else if (c.dense_M > 0) {
      f.row0 = mt * S::BM;
      f.rows = static_cast<int>(min(static_cast<int64_t>(S::BM), c.dense_M - f.row0));
      f.grp = 0;
    } else {
      f.row0 = c.tiles.row0[mt];
      f.rows = c.tiles.rows[mt];
      f.grp = c.tiles.expert[mt];
    }
#pragma unroll
    for (int q = 0; q < S::NQ; ++q) {
      f.src[q] = 0;
      const int i = wave + S::NW * q;
      // (the first condition is known at compile time: loads past it read weight rows)
      if (S::NW * q >= S::BM / S::kRowsPerDma || !load_is_a(q) || TA) continue;
      const int r = i * S::kRowsPerDma + dma_row;
      int64_t p = f.row0 + (r < f.rows ? r : 0);
      p = min(max(p, int64_t(0)), c.rows_bound - 1);
      f.src[q] = static_cast<int32_t>(GATHER ? static_cast<int64_t>(c.gather[p]) / c.gather_div : p);
    }
    f.scsrc = 0;
    if constexpr (S::MX) {
      const int r = wave * 64 + lane;
      if (wave < S::NSC && r < S::BM) {
        int64_t p = f.row0 + (r < f.rows ? r : 0);
        p = min(max(p, int64_t(0)), c.rows_bound - 1);
        f.scsrc = static_cast<int32_t>(GATHER ? static_cast<int64_t>(c.gather[p]) / c.gather_div : p);
      }
    }
  };

  // The tile's load offsets from what fetch() read (registers only).
  auto setup_fetched = [&](const TileFetch& f, TileState& t) {
    t.nt = f.nt;
    t.row0 = f.row0;
    t.rows = f.rows;
    const int64_t grp = f.grp;
    t.nk = static_cast<int>(c.Kd / S::BK);
    t.kcnt = 0;
    t.cofs = 0;
    t.Abase = Ab;
    if (WGRAD) {
      t.kcnt = f.kcnt;
      t.nk = (t.kcnt + S::BK - 1) / S::BK;
      t.cofs = grp * c.c_group_stride;
      t.Abase = Ab + f.kb * c.lda * 2;
      t.Bexp = static_cast<const unsigned char*>(c.B) + f.kb * c.ldb * 2;
    } else {
      t.Bexp = static_cast<const unsigned char*>(c.B) + grp * c.b_group_stride * S::EB;
    }
#pragma unroll
    for (int q = 0; q < S::NQ; ++q) {
      const int i = wave + S::NW * q;
      const bool is_a = load_is_a(q);
      if ((is_a && TA) || (!is_a && TB)) {
        // contraction-major: this lane fetches 16 bytes of staged row tr (contraction index),
        // logical chunk tc, into the linear DMA slot
        const int il = is_a ? i : i - S::BM / S::kRowsPerDma;
        const int tr = 2 * il + (lane >> 5);
        const int tc = (lane & 31) ^ ((tr & 3) << 2);
        const int64_t width = is_a ? c.dense_M : c.N;    // columns of the operand
        const int64_t col0 = is_a ? t.row0 : t.nt * S::BN;
        const int64_t col = min(col0 + 8 * tc, width - 8);
        t.src_off[q] = static_cast<uint32_t>((tr * (is_a ? c.lda : c.ldb) + col) * 2);
        continue;
      }
      const int r = (is_a ? i : i - S::BM / S::kRowsPerDma) * S::kRowsPerDma + dma_row;
      // the logical chunk this lane fetches, so that the linear LDS write lands swizzled
      const int chunk_l = (lane % S::CHUNKS) ^ ((r / S::ROWS_PER_BANKLINE) & (S::CHUNKS - 1));
      if (is_a) {
        const int64_t src = min(max(static_cast<int64_t>(f.src[q]), int64_t(0)), c.a_rows - 1);
        t.src_off[q] = static_cast<uint32_t>(src * c.lda * S::EB + chunk_l * 16);
      } else {
        int64_t wrow;
        // weight rows of plane p follow those of plane p-1
        const int plane = S::PLANES == 1 ? 0 : r / S::BN, rp = S::PLANES == 1 ? r : r % S::BN;
        if (SWIGLU) {
          const int wv = rp / (S::TN * 32), qq = rp % (S::TN * 32);
          const int half = qq / (S::TN * 16);
          int64_t col = t.nt * (S::BN / 2) + wv * (S::TN * 16) + (qq % (S::TN * 16));
          col = min(col, c.N - 1);
          wrow = col + (half ? c.swiglu_h : 0);
        } else {
          wrow = min(t.nt * S::BN + rp, c.N - 1);
        }
        const int64_t pbase = S::PLANES == 1 ? 0 : plane * c.b_plane_stride;
        t.src_off[q] = static_cast<uint32_t>((pbase + wrow * c.ldb) * S::EB + chunk_l * 16);
      }
    }
    if constexpr (S::MX) {
      // wavefront w < NSC loads the scales of staged rows [64 w, 64 w + 64): token rows first,
      // then weight rows, the same rows (and padding clamps) as the operand loads above
      if (wave < S::NSC) {
        const int r = wave * 64 + lane;
        if (r < S::BM) {
          const int64_t src = min(max(static_cast<int64_t>(f.scsrc), int64_t(0)), c.a_rows - 1);
          t.sc_base = c.a_scale;
          t.sc_off = static_cast<uint32_t>(src * c.a_scale_ld);
        } else {
          const int rp = r - S::BM;
          int64_t wrow;
          if (SWIGLU) {
            const int wv = rp / (S::TN * 32), qq = rp % (S::TN * 32);
            const int half = qq / (S::TN * 16);
            int64_t col = t.nt * (S::BN / 2) + wv * (S::TN * 16) + (qq % (S::TN * 16));
            col = min(col, c.N - 1);
            wrow = col + (half ? c.swiglu_h : 0);
          } else {
            wrow = min(t.nt * S::BN + rp, c.N - 1);
          }
          t.sc_base = c.b_scale + grp * c.b_scale_group_stride;
          t.sc_off = static_cast<uint32_t>(wrow * c.b_scale_ld);
        }
      }
    }
  };

  auto setup = [&](int64_t it, TileState& t) {
    TileFetch f;
    fetch(it, f);
    setup_fetched(f, t);
  };

  // Every operand loads through buffer descriptors (buffer_load ... lds) with uniform bases, so
  // a stage's loads need no per-lane address arithmetic. Row-major operands and contraction-major
  // weights: one descriptor per operand and tile, the k-stage step a scalar offset. Weight-
  // gradient operands (contraction over a group's rows): the descriptor moves to the stage's first
  // contraction row and its range ends at the group's last row, so rows past the group read as
  // zeros (an out-of-range buffer load returns zero; the range check covers the per-lane offset,
  // which therefore carries no k-stage step).
  // DMA loads of k-stage kt of tile t into ring slot `st` (lds0 or lds1).
  auto issue = [&](const TileState& t, int kt, unsigned char* st) {
#if defined(__HIP_DEVICE_COMPILE__)
    // bases and ranges are uniform; readfirstlane keeps them in scalar registers
    auto rsrc = [](const unsigned char* p, uint32_t bytes) {
      const uint64_t v = reinterpret_cast<uint64_t>(p);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
      const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
      return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo),
                                               static_cast<short>(0), static_cast<int>(n), 0x00020000);
    };
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t soa, sob;
    if constexpr (WGRAD) {
      const uint32_t da = static_cast<uint32_t>(kt) * a_step, db = static_cast<uint32_t>(kt) * b_step;
      const int64_t la = static_cast<int64_t>(t.kcnt) * c.lda * 2 - da;
      const int64_t lb = static_cast<int64_t>(t.kcnt) * c.ldb * 2 - db;
      ra = rsrc(t.Abase + da, la > 0 ? static_cast<uint32_t>(la) : 0u);
      rb = rsrc(t.Bexp + db, lb > 0 ? static_cast<uint32_t>(lb) : 0u);
      soa = 0;
      sob = 0;
    } else {
      // no range limit (every offset is below 4 GiB): row indices are clamped where they are made
      ra = rsrc(Ab, 0xFFFFFFFFu);
      rb = rsrc(t.Bexp, 0xFFFFFFFFu);
      soa = static_cast<uint32_t>(kt) * a_step;
      sob = static_cast<uint32_t>(kt) * b_step;
    }
#endif
#pragma unroll
    for (int q = 0; q < S::NQ; ++q) {
      const int i = wave + S::NW * q;
      if (S::NI % S::NW != 0 && i >= S::NI) continue;
      const bool is_a = load_is_a(q);
      // Small tiles (few rows per expert): token rows past the tile's last valid row are never
      // stored, so their loads are skipped (whatever LDS holds there only feeds output rows
      // that are dropped). The large tiles keep every load: the extra live register spills.
      if (S::BM < 256 && !TA && !WGRAD && is_a && i * S::kRowsPerDma >= t.rows) continue;
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb, LDS_PTR(st + i * 1024), 16, t.src_off[q],
                                               is_a ? soa : sob, 0, 0);
#endif
    }
    if constexpr (S::SCG == 1) {
      if (wave < S::NSC)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(t.sc_base + (t.sc_off + static_cast<uint32_t>(kt) * 4)),
                                         LDS_PTR(st + S::DATA + wave * 256), 4, 0, 0);
    } else if constexpr (S::SCG == 4) {
      // Stage kt's loads land before stage kt runs; group kt / 4 goes to the half that group
      // kt / 4 - 2 used, whose last reader (stage kt - 5) every wavefront has passed.
      if (wave < S::NSC && (kt & 3) == 0)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(t.sc_base + (t.sc_off + static_cast<uint32_t>(kt) * 4)),
                                         LDS_PTR(ldssc + ((kt >> 2) & 1) * S::SCHALF + wave * 1024),
                                         16, 0, 0);
    }
  };

  f32x16 acc[S::TM][S::TN];
  bf16x8 fw[S::MX ? 1 : 2][S::PLANES][S::TN], ft[S::MX ? 1 : 2][S::TM];
  // MXFP8 operands: 32 codes per lane (two 16-byte chunks: the lane's halves of the two
  // 32-element blocks of a 64-k step) and the scale words of the stage
  i32x8 fwx[S::MX ? 2 : 1][S::TN], ftx[S::MX ? 2 : 1][S::TM];
  uint32_t scw[S::TN], sct[S::TM];
  auto lds_frags_mx = [&](int fs, const unsigned char* la, const unsigned char* lb, int kk) {
    const int c0 = 4 * kk + (lane >> 5), c1 = c0 + 2;
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      const int row = wn * S::TN * 32 + j * 32 + (lane & 31);
      const u32x4v lo = *reinterpret_cast<const u32x4v*>(lb + swz<S>(row, c0));
      const u32x4v hi = *reinterpret_cast<const u32x4v*>(lb + swz<S>(row, c1));
      fwx[fs][j] = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]), static_cast<int>(lo[3]),
                         static_cast<int>(hi[0]), static_cast<int>(hi[1]), static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    }
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int row = wm * S::TM * 32 + i * 32 + (lane & 31);
      const u32x4v lo = *reinterpret_cast<const u32x4v*>(la + swz<S>(row, c0));
      const u32x4v hi = *reinterpret_cast<const u32x4v*>(la + swz<S>(row, c1));
      ftx[fs][i] = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]), static_cast<int>(lo[3]),
                         static_cast<int>(hi[0]), static_cast<int>(hi[1]), static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    }
  };
  // scale bytes [b0 b1 b2 b3] of the stage's four blocks, shifted so that byte 0 is block
  // (lane / 32) (64-k step 0) and byte 2 block 2 + (lane / 32) (step 1)
  // (scl: the stage's scale words, rstride bytes apart per staged row)
  auto lds_scales = [&](const unsigned char* scl, int rstride) {
    const int shift = 8 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
      scw[j] = *reinterpret_cast<const uint32_t*>(scl + (S::BM + wn * S::TN * 32 + j * 32 + (lane & 31)) * rstride) >> shift;
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
      sct[i] = *reinterpret_cast<const uint32_t*>(scl + (wm * S::TM * 32 + i * 32 + (lane & 31)) * rstride) >> shift;
  };
  auto lds_frags = [&](int fs, const unsigned char* la, const unsigned char* lb, int kk) {
    const int ch = 2 * kk + (lane >> 5);
#pragma unroll
    for (int pl = 0; pl < S::PLANES; ++pl)
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
        if constexpr (TB)
          fw[fs][pl][j] = tr_frag(lb, wn * S::TN * 32 + j * 32, kk, lane);
        else
          fw[fs][pl][j] = *reinterpret_cast<const bf16x8*>(
              lb + swz<S>(pl * S::BN + wn * S::TN * 32 + j * 32 + (lane & 31), ch));
      }
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      if constexpr (TA)
        ft[fs][i] = tr_frag(la, wm * S::TM * 32 + i * 32, kk, lane);
      else
        ft[fs][i] = *reinterpret_cast<const bf16x8*>(la + swz<S>(wm * S::TM * 32 + i * 32 + (lane & 31), ch));
    }
  };

  // Epilogue, staged through LDS slot 1 (slot 0 is receiving the next tile's first stage).
  // Lane holds token row (lane & 31) of each 32-row sub-tile and weight rows
  // 8*g + 4*(lane >> 5) + {0..3} of each 32-row weight sub-tile (g = 0..3), i.e. 8 bytes of
  // 32 different output rows per register group: stored directly that is 32 partial lines per
  // instruction. Instead the tile goes to LDS in bf16 and leaves as whole rows, every store
  // instruction writing full 128-byte lines. The output tile (BM x OUTC bf16) passes in NR
  // rounds of RR rows; round rho carries sub-tiles i in [rho*TMR, (rho+1)*TMR) of every wavefront.
  constexpr int OUTC = SWIGLU ? S::BN / 2 : S::BN;      // output columns per tile
  constexpr int EB = static_cast<int>(sizeof(OutT));    // bytes per output element
  constexpr int EPC = 16 / EB;                          // output elements per 16-byte chunk
  constexpr int RB = OUTC * EB;                         // bytes per output row
  constexpr int CPR = RB / 16;                          // 16-byte chunks per output row
  constexpr int NR = (S::BM * RB + S::STAGE - 1) / S::STAGE;
  constexpr int TMR = S::TM / NR;
  constexpr int RR = S::BM / NR;                        // rows per round
  constexpr int RPI = S::NT * 16 / RB;                  // rows per store instruction
  constexpr int KI = RR / RPI;                          // store instructions per thread per round
  static_assert(S::TM % NR == 0 && RR % RPI == 0 && RR * RB <= S::STAGE, "epilogue staging");
  unsigned char* stg = lds1;
  // LDS byte address of byte b of staged row lr: 16-byte chunks XOR-swizzled by row, so the
  // 32 rows of one register group land in distinct bank groups and a row read stays whole.
  auto stg_addr = [&](int lr, int b) {
    return lr * RB + ((((b >> 4) ^ (lr & (CPR - 1))) << 4) | (b & 15));
  };
  // tile row of staged row lr in round rho
  auto tile_row = [&](int rho, int lr) {
    const int w = lr / (TMR * 32), ii = (lr % (TMR * 32)) / 32;
    return w * S::TM * 32 + (rho * TMR + ii) * 32 + (lr & 31);
  };
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  // Epilogue of tile t. When `more`, stage 0 of tile nx is issued into slot 0 once slot 1 holds
  // the last staging round: its loads then overlap the last round's reads and stores. (Issued
  // earlier, the compiler would wait for them before the staging writes, which share LDS.)
  // Large tiles issue the next tile's first stage as soon as the epilogue starts (its list
  // entry and row indices were fetched during this tile's k-loop), so those loads overlap the
  // whole epilogue; they fill ring slot 0 while the epilogue stages through slot 1. There every
  // wavefront issues exactly NQ operand loads (plus one scale load for MXFP8 wavefronts below
  // NSC), the count the scatter wait below relies on. Other shapes issue it in the last round.
  constexpr bool EARLY = !WGRAD && !S::MX && S::BM == 256 && S::NI % S::NW == 0;
  // Large tiles (and the weight-gradient tiles) stagger their loads (see the k-loop): every
  // k-stage issues its loads, the last one of a tile reloading its own stage into the free slot,
  // so the epilogue first waits for those before it reuses a slot.
  constexpr bool STAGGER = EARLY || WGRAD;
  constexpr int NSIDX = SCATTER ? (EARLY ? NR * KI : KI) : 1;
  auto epilogue = [&](const TileState& t, bool more, const TileFetch& fn, int64_t it_next, TileState& nx) {
    // The thread index passes through an empty asm statement: the epilogue's per-lane addresses
    // are then computed here, not hoisted out of the persistent loop, where they would hold
    // registers through every k-stage.
    int etid = tid;
    asm volatile("" : "+v"(etid));
    const int elane = etid & 63;
    const int quad = 4 * (elane >> 5);
    const int64_t col0 = t.nt * OUTC;
    // Scatter indices of the rows this thread stores in round rho (all rounds up front when the
    // next tile's loads follow them), fetched first so their latency overlaps the LDS round trip.
    int sidx[NSIDX];
    auto load_sidx = [&](int rho, int base) {
#pragma unroll
      for (int k = 0; k < KI; ++k) {
        const int m = tile_row(rho, k * RPI + etid / CPR);
        sidx[base + k] = c.scatter[min(t.row0 + (m < t.rows ? m : 0), c.rows_bound - 1)];
      }
    };
    if constexpr (STAGGER) wait_vmcnt<0>();
    if constexpr (SCATTER && EARLY) {
#pragma unroll
      for (int rho = 0; rho < NR; ++rho) load_sidx(rho, rho * KI);
    }
    if constexpr (EARLY) {
      // The same loads are in flight after the indices on every path: with no next tile the
      // current tile's first stage is loaded again (valid addresses, into the free slot 0,
      // never read; the exit waits for it).
      if (more) {
        setup_fetched(fn, nx);
        issue(nx, 0, lds0);
      } else {
        issue(t, 0, lds0);
      }
    }
#pragma unroll
    for (int rho = 0; rho < NR; ++rho) {
      if constexpr (SCATTER && !EARLY) load_sidx(rho, 0);
      if (rho > 0) {  // every wavefront done reading the previous round
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
      }
#pragma unroll
      for (int ii = 0; ii < TMR; ++ii) {
        const int i = rho * TMR + ii;
        const int lr = wm * TMR * 32 + ii * 32 + (elane & 31);
        if (SWIGLU) {
#pragma unroll
          for (int j = 0; j < S::TN / 2; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              uint16_t o[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float up = acc[i][j][4 * g + r];
                const float gate = acc[i][j + S::TN / 2][4 * g + r];
                // silu(gate) = gate / (1 + 2^(-gate * log2 e)): hardware exp2 and reciprocal,
                // a few fp32 ulp, far below the bf16 rounding that follows
                const float e = __builtin_amdgcn_exp2f(-gate * 1.44269504088896340736f);
                o[r] = f32_to_bf16_bits(up * gate * __builtin_amdgcn_rcpf(1.f + e));
              }
              const int ct = wn * (S::TN * 16) + j * 32 + 8 * g + quad;
              if constexpr (H_OUT) {
                // training forward: the pre-activation H (bf16, [up | gate]) of this lane's
                // 4 columns, stored straight from the registers
                const int m = wm * S::TM * 32 + i * 32 + (elane & 31);
                const int64_t hc = col0 + ct;
                if (m < t.rows && hc < c.N) {
                  uint16_t* hr = static_cast<uint16_t*>(c.h_out) + min(t.row0 + m, c.rows_bound - 1) * 2 * c.swiglu_h;
                  uint32_t u[2], gv[2];
#pragma unroll
                  for (int r = 0; r < 2; ++r) {
                    u[r] = f32_to_bf16_bits(acc[i][j][4 * g + 2 * r]) |
                           (static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * g + 2 * r + 1])) << 16);
                    gv[r] = f32_to_bf16_bits(acc[i][j + S::TN / 2][4 * g + 2 * r]) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j + S::TN / 2][4 * g + 2 * r + 1])) << 16);
                  }
                  *reinterpret_cast<uint2*>(hr + hc) = make_uint2(u[0], u[1]);
                  *reinterpret_cast<uint2*>(hr + c.swiglu_h + hc) = make_uint2(gv[0], gv[1]);
                }
              }
              lds_store_b64(stg + stg_addr(lr, ct * 2), o[0] | (static_cast<uint32_t>(o[1]) << 16),
                            o[2] | (static_cast<uint32_t>(o[3]) << 16));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < S::TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int ct = wn * (S::TN * 32) + j * 32 + 8 * g + quad;
              if constexpr (OUT_F32) {
                lds_store_b128(stg + stg_addr(lr, ct * 4), acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                               acc[i][j][4 * g + 3]);
              } else {
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = f32_to_bf16_bits(acc[i][j][4 * g + r]);
                lds_store_b64(stg + stg_addr(lr, ct * 2), o[0] | (static_cast<uint32_t>(o[1]) << 16),
                              o[2] | (static_cast<uint32_t>(o[3]) << 16));
              }
            }
          }
        }
      }
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      // The scatter indices of this round (loaded at its start) are waited for once here; left
      // to the compiler, every store would wait for all vector-memory operations in flight
      // (the next tile's first loads and the previous stores) before using its index.
      // (EARLY: only the next tile's loads were issued after the indices, and loads complete
      // in order, so waiting until that many remain in flight is enough.)
      if constexpr (SCATTER) {
        if constexpr (EARLY) {
          if (rho == 0) {
            // Once they have landed the indices pass through an empty asm statement: they are
            // then no longer load results to the compiler, which would otherwise wait for every
            // load in flight (the next tile's too) before each store.
            static_assert(!EARLY || !S::MX, "the wait below counts operand loads only");
            wait_vmcnt<S::NQ>();
#pragma unroll
            for (int k = 0; k < NSIDX; ++k) asm volatile("" : "+v"(sidx[k]));
          }
        } else {
          wait_vmcnt<0>();
        }
      }
      const int cc = etid % CPR;
      const int64_t col = col0 + cc * EPC;
      u32x4_t v[KI];
#pragma unroll
      for (int k = 0; k < KI; ++k) v[k] = *reinterpret_cast<const u32x4_t*>(stg + stg_addr(k * RPI + etid / CPR, cc * 16));
      // Other shapes: the accumulators are dead once the last round is in LDS; set up the next
      // tile then (its index loads, then its first DMA loads, ahead of this round's stores).
      if constexpr (!EARLY) {
        if (rho == NR - 1 && more) {
          setup(it_next, nx);
          if (!WGRAD || nx.nk > 0) issue(nx, 0, lds0);
        }
      }
#pragma unroll
      for (int k = 0; k < KI; ++k) {
        const int lr = k * RPI + etid / CPR;
        const int m = tile_row(rho, lr);
        const int64_t orow = SCATTER ? static_cast<int64_t>(sidx[SCATTER ? (EARLY ? rho * KI : 0) + k : 0]) : t.row0 + m;
        if constexpr (SWIGLU_BWD) {
          // v holds 8 columns of d_act (bf16) of sorted row orow; with the saved up / gate of
          // those columns: d_up = d_act * silu(gate), d_gate = d_act * up * silu'(gate),
          // silu' = sigmoid * (1 + gate * (1 - sigmoid)), in fp32, stored as bf16.
          if (m < t.rows && col < c.N) {
            const int64_t p = min(max(orow, int64_t(0)), c.rows_bound - 1);
            const uint16_t* hr = static_cast<const uint16_t*>(c.h_in) + p * 2 * c.bwd_h;
            const u32x4_t hu = *reinterpret_cast<const u32x4_t*>(hr + col);
            const u32x4_t hg = *reinterpret_cast<const u32x4_t*>(hr + c.bwd_h + col);
            u32x4_t du, dg;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              uint32_t ou[2], og[2];
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const float d = __uint_as_float(hh ? (v[k][w] & 0xFFFF0000u) : (v[k][w] << 16));
                const float up = __uint_as_float(hh ? (hu[w] & 0xFFFF0000u) : (hu[w] << 16));
                const float gate = __uint_as_float(hh ? (hg[w] & 0xFFFF0000u) : (hg[w] << 16));
                const float e = __builtin_amdgcn_exp2f(-gate * 1.44269504088896340736f);
                const float sig = __builtin_amdgcn_rcpf(1.f + e);
                ou[hh] = f32_to_bf16_bits(d * (gate * sig));
                og[hh] = f32_to_bf16_bits(d * up * (sig * (1.f + gate * (1.f - sig))));
              }
              du[w] = ou[0] | (ou[1] << 16);
              dg[w] = og[0] | (og[1] << 16);
            }
            uint16_t* dr = reinterpret_cast<uint16_t*>(Cbase) + p * c.ldc;
            *reinterpret_cast<u32x4_t*>(dr + col) = du;
            *reinterpret_cast<u32x4_t*>(dr + c.bwd_h + col) = dg;
          }
        } else if constexpr (OUT_MX) {
          // MXFP8 output (the bf16 values staged above, quantised as the standalone quantiser
          // does): a 32-column block is the 16-byte chunks of 4 adjacent lanes of one row;
          // its amax comes from two lane exchanges inside the group, executed by every lane.
          float x[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(v[k][i] << 16);
            x[2 * i + 1] = __uint_as_float(v[k][i] & 0xFFFF0000u);
          }
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
          amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
          amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
          const int sc = mx_scale_code(amax), sh = 127 - sc;
          const uint32_t q0 = pack4_e4m3(ldexpf(x[0], sh), ldexpf(x[1], sh), ldexpf(x[2], sh), ldexpf(x[3], sh));
          const uint32_t q1 = pack4_e4m3(ldexpf(x[4], sh), ldexpf(x[5], sh), ldexpf(x[6], sh), ldexpf(x[7], sh));
          if (m < t.rows && col < c.N) {
            const int64_t r = min(max(orow, int64_t(0)), c.c_rows - 1);
            *reinterpret_cast<uint2*>(c.c_codes + r * c.ldc + col) = make_uint2(q0, q1);
            if ((cc & 3) == 0) c.c_scales[r * (c.N / 32) + col / 32] = static_cast<uint8_t>(sc);
          }
        } else {
          // Non-temporal: every CU writes its tile in the same burst at the end of a round of
          // tiles; streaming the rows past the caches keeps the operand lines the next tiles read.
          if (m < t.rows && col < c.N)
            __builtin_nontemporal_store(
                v[k], reinterpret_cast<u32x4_t*>(Cbase + (WGRAD ? t.cofs : 0) +
                                                 min(max(orow, int64_t(0)), c.c_rows - 1) * c.ldc + col));
        }
      }
    }
  };

  // Persistent loop over this workgroup's tiles: it = slot, slot + per_xcd, ... inside the
  // XCD's chunk. Stage 0 of the next tile is issued before the current tile's epilogue, so its
  // load latency hides under the epilogue's stores.
  // Weight-gradient tiles differ in cost (a group's contraction is its row count), so they are
  // handed out instead: thread 0 takes the next index from the zeroed tile counter when a tile
  // starts and passes it through LDS (two slots, alternating: a slot is rewritten two tiles
  // later, after barriers every wavefront has passed); the sequence puts the largest groups
  // first. Every workgroup leaves once the counter passes the last tile.
  int32_t* sched = nullptr;
  if constexpr (WGRAD) {
    __shared__ int32_t s_sched[2];
    sched = s_sched;
    if (tid == 0) s_sched[0] = atomicAdd(c.tile_counter, 1);
    __syncthreads();
  }
  // Other modes: it is the tile's position in the linear sequence; this workgroup's tiles are
  // those from its first in steps of it_step below lin_end.
  const int64_t slot = blockIdx.x / kXcds;
  const int64_t lin_end = SP ? total : min(total, (xcd + 1) * chunk);
  const int64_t it_step = (SP ? kXcds : 1) * static_cast<int64_t>(per_xcd);
  int64_t it = WGRAD ? static_cast<int64_t>(sched[0]) : (SP ? xcd + slot * kXcds : xcd * chunk + slot);
  if (WGRAD ? it >= total : (slot >= per_xcd || it >= lin_end)) return;
  int parity = 1;
  TileFetch fnext;
  TileState cur;
  setup(it, cur);
  if (!WGRAD || cur.nk > 0) issue(cur, 0, lds0);
  for (;;) {
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (WGRAD && tid == 0) sched[parity] = atomicAdd(c.tile_counter, 1);
    const int nk = WGRAD ? cur.nk : static_cast<int>(c.Kd / S::BK);
    // EARLY: the next tile of this workgroup's sequence, fetched during the first stage
    const int64_t it_pre = it + it_step;
    const bool fetch_next = EARLY && it_pre < lin_end;
    if (fetch_next && nk <= 0) fetch(it_pre, fnext);
    // The MFMA work of k-stage kt from slot `la`, with its scheduling directives. late
    // (staggered loads, see the k-loop below): this wavefront's loads of the stage come after
    // its first k16 step instead of before its first LDS reads.
    auto stage_compute = [&](int kt, const unsigned char* la, auto late) __attribute__((always_inline)) {
      const unsigned char* lb = la + S::BM * S::ROWB;
      // k16 steps with fragments double-buffered in registers; the directives interleave step
      // kk+1's LDS reads with step kk's MFMAs so the matrix pipe does not wait on an LDS round
      // trip before every MFMA group.
      if constexpr (S::MX) {
        // two 64-k steps per 128-element stage; scale words read once per stage
        if constexpr (S::SCG == 1)
          lds_scales(la + S::DATA, 4);
        else
          lds_scales(ldssc + ((kt >> 2) & 1) * S::SCHALF + (kt & 3) * 4, 16);
        lds_frags_mx(0, la, lb, 0);
#pragma unroll
        for (int kk = 0; kk < S::BK / 64; ++kk) {
          if (kk + 1 < S::BK / 64) lds_frags_mx((kk + 1) & 1, la, lb, kk + 1);
#pragma unroll
          for (int i = 0; i < S::TM; ++i)
#pragma unroll
            for (int j = 0; j < S::TN; ++j)
              acc[i][j] = mfma_mx(fwx[kk & 1][j], ftx[kk & 1][i], acc[i][j], scw[j] >> (16 * kk), sct[i] >> (16 * kk));
        }
      } else {
        constexpr int kSteps = S::BK / 16;
        // LDS fragment reads per k16 step (a contraction-major fragment takes two)
        constexpr int kReads = (TA ? 2 : 1) * S::TM + (TB ? 2 : 1) * S::PLANES * S::TN;
        constexpr int kMfma = S::TM * S::TN * S::PLANES;   // MFMAs per k16 step
        lds_frags(0, la, lb, 0);
#pragma unroll
        for (int kk = 0; kk < kSteps; ++kk) {
          if (kk + 1 < kSteps) lds_frags((kk + 1) & 1, la, lb, kk + 1);
#pragma unroll
          for (int i = 0; i < S::TM; ++i)
#pragma unroll
            for (int j = 0; j < S::TN; ++j)
#pragma unroll
              for (int pl = S::PLANES - 1; pl >= 0; --pl)  // smallest plane first
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[kk & 1][pl][j], ft[kk & 1][i], acc[i][j], 0, 0, 0);
        }
        if constexpr (STAGGER)
          sched_stage_loads_at<kSteps, kReads, kMfma, S::NQ, decltype(late)::value ? 0 : -1>();
        else
          sched_stage<kSteps, kReads, kMfma, 0>();
      }
    };
    // Stage kt reads slot `la` (lds0 for even kt, lds1 for odd) and refills the other one; the
    // loop runs two stages per iteration so that each stage's slot is known at compile time.
    auto kstage = [&](int kt, const unsigned char* la, unsigned char* other) {
      // This wavefront's loads of stage kt have landed; after the barrier so have every
      // wavefront's, and every wavefront is done reading stage kt-1, whose slot is refilled.
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (kt + 1 < nk) issue(cur, kt + 1, other);
      if (fetch_next && kt == 0) fetch(it_pre, fnext);
      stage_compute(kt, la, std::false_type{});
    };
    // The same with staggered loads: every stage issues its loads unconditionally, so they sit in
    // the MFMAs' block where the directives place them; the last stage of a tile reloads its own
    // stage into the free slot (valid addresses, never read), which the epilogue waits for.
    auto kstage_staggered = [&](int kt, const unsigned char* la, unsigned char* other, auto late)
                                __attribute__((always_inline)) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      issue(cur, kt + 1 < nk ? kt + 1 : kt, other);
      stage_compute(kt, la, late);
      if (fetch_next && kt == 0) fetch(it_pre, fnext);
    };
    // A stage's 64 loads issued as one burst right after the barrier fill the address unit's
    // queues, and a wavefront stalls on issue before it reaches its MFMAs. With STAGGER the two
    // wavefronts of a SIMD (w and w + 4) split: the first half issues at the stage start, the
    // second after its first k16 step, so one of each pair computes while the other's loads
    // queue. (Same-box A/B, outputs bitwise equal: skewed layer 11.90 -> 11.58 ms, olmoe -2 %,
    // latent896 -1 %; the second half one step later, or its loads interleaved with the MFMAs,
    // measured slower.)
    if constexpr (STAGGER) {
      auto kloop = [&](auto late) __attribute__((always_inline)) {
        for (int kt = 0; kt < nk; kt += 2) {
          kstage_staggered(kt, lds0, lds1, late);
          if (kt + 1 < nk) kstage_staggered(kt + 1, lds1, lds0, late);
        }
      };
      if (wave >= S::NW / 2)
        kloop(std::true_type{});
      else
        kloop(std::false_type{});
    } else {
      for (int kt = 0; kt < nk; kt += 2) {
        kstage(kt, lds0, lds1);
        if (kt + 1 < nk) kstage(kt + 1, lds1, lds0);
      }
    }
    // Every wavefront done reading this tile's last stages: slot 0 is free for the next tile.
    // (Weight-gradient mode: a full workgroup barrier with fences, which also publishes the
    // next tile index thread 0 wrote to LDS; no vector-memory load is in flight here.)
    if constexpr (WGRAD) {
      __syncthreads();
    } else {
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
    }

    int64_t it_next;
    bool more;
    if constexpr (WGRAD) {
      it_next = sched[parity];  // written at this tile's start, before the barrier above
      more = it_next < total;
      parity ^= 1;
    } else {
      it_next = it + it_step;
      more = it_next < lin_end;
    }
    TileState nxt;
    epilogue(cur, more, fnext, it_next, nxt);
    if (!more) break;
    cur = nxt;
    it = it_next;
  }
  // Nothing is left in flight that writes LDS (each tile's last stage issues no refill and the
  // last tile issues no next stage), but keep the invariant explicit before LDS is released.
  wait_vmcnt<0>();
}

// TRANS: bit 0 = the token operand A is contraction-major, bit 1 = the weight operand B is (see
// GemmCall::trans). WGRAD: weight-gradient mode, the contraction runs over each group's rows
// (GemmCall::group_offsets). SWIGLU_BWD: the SwiGLU-backward epilogue (GemmCall::bwd_h).
// H_OUT: the SwiGLU epilogue also stores the pre-activation (GemmCall::h_out).
// Grouped products over a marked tile list run the spread tile order. The body is compiled once
// per order, so neither copy keeps the other's loop bounds live (the large tiles have no
// registers to spare); weight-gradient kernels, whose tiles are handed out, have one copy.
template <class S, bool SWIGLU, bool GATHER, bool SCATTER, bool OUT_F32 = false, bool OUT_MX = false, int TRANS = 0,
          bool WGRAD = false, bool SWIGLU_BWD = false, bool H_OUT = false>
__global__ __launch_bounds__(S::NT) __attribute__((amdgpu_waves_per_eu(2))) void gemm_bf16_kernel(GemmCall c) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[S::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[S::STAGE];
  constexpr bool kSpreadable = !WGRAD;
  if constexpr (kSpreadable) {
    if (c.dense_M <= 0 && c.tiles.count[1] != 0) {
      gemm_bf16_body<S, SWIGLU, GATHER, SCATTER, OUT_F32, OUT_MX, TRANS, WGRAD, SWIGLU_BWD, H_OUT, true>(c, lds0, lds1);
      return;
    }
  }
  gemm_bf16_body<S, SWIGLU, GATHER, SCATTER, OUT_F32, OUT_MX, TRANS, WGRAD, SWIGLU_BWD, H_OUT, false>(c, lds0, lds1);
}

template <class S>
int64_t persistent_grid(const GemmCall& c, int wg_per_cu) {
  const int64_t cols_per_tile = c.swiglu_h > 0 ? S::BN / 2 : S::BN;
  const int64_t ntn = (c.N + cols_per_tile - 1) / cols_per_tile;
  const int64_t tiles_upper = c.dense_M > 0 ? ((c.dense_M + S::BM - 1) / S::BM) * ntn
                                            : static_cast<int64_t>(c.tiles.cap) * ntn;
  if (tiles_upper <= 0 || c.rows_bound <= 0) return 0;
  const int64_t grid = std::min<int64_t>(tiles_upper, static_cast<int64_t>(device_cu_count()) * wg_per_cu);
  return ((grid + kXcds - 1) / kXcds) * kXcds;  // whole XCD rounds
}

template <class S>
hipError_t launch_shape(const GemmCall& c, hipStream_t s, int wg_per_cu) {
  const int64_t cols_per_tile = c.swiglu_h > 0 ? S::BN / 2 : S::BN;
  const int64_t ntn = (c.N + cols_per_tile - 1) / cols_per_tile;
  const int64_t tiles_upper = c.dense_M > 0 ? ((c.dense_M + S::BM - 1) / S::BM) * ntn
                                            : static_cast<int64_t>(c.tiles.cap) * ntn;
  if (tiles_upper <= 0 || c.rows_bound <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(tiles_upper, static_cast<int64_t>(device_cu_count()) * wg_per_cu);
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;  // whole XCD rounds
  const dim3 g(static_cast<unsigned>(grid)), b(S::NT);
  const bool sw = c.swiglu_h > 0, ga = c.gather != nullptr, sc = c.scatter != nullptr;
  if (c.h_out && !(sw && ga && !sc && !S::MX)) return hipErrorInvalidValue;
  if (sw && ga && !sc && c.h_out) {
    if constexpr (!S::MX)
      hipLaunchKernelGGL((gemm_bf16_kernel<S, true, true, false, false, false, 0, false, false, true>), g, b, 0, s, c);
  } else if (sw && ga && !sc) hipLaunchKernelGGL((gemm_bf16_kernel<S, true, true, false>), g, b, 0, s, c);
  else if (!sw && !ga && sc) hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, true>), g, b, 0, s, c);
  else if (!sw && !ga && !sc) hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, false>), g, b, 0, s, c);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

int gemm_bf16_tile_m(int variant) { return variant == 0 ? ShapeLarge::BM : ShapeSmall::BM; }

int gemm_bf16_round_tiles() {
  const int64_t g = static_cast<int64_t>(device_cu_count()) * ShapeLarge::WG_PER_CU;
  return static_cast<int>(((g + kXcds - 1) / kXcds) * kXcds);  // whole XCD rounds, as launched
}

int gemm_bf16_swiglu_tile_cols() { return ShapeLarge::BN / 2; }

int gemm_bf16_planes_tile_n() { return ShapeRouter::BN; }

hipError_t launch_gemm_bf16_planes_f32(const GemmCall& c, hipStream_t s) {
  // dense fp32 output only: no gather, scatter, SwiGLU or expert groups
  if (c.dense_M <= 0 || c.gather || c.scatter || c.swiglu_h > 0 || c.N % 4 != 0) return hipErrorInvalidValue;
  const int64_t grid = persistent_grid<ShapeRouter>(c, ShapeRouter::WG_PER_CU);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<ShapeRouter, false, false, false, true>), dim3(static_cast<unsigned>(grid)),
                     dim3(ShapeRouter::NT), 0, s, c);
  return hipGetLastError();
}

int gemm_bf16_pick_variant(double mean_rows_per_group) { return mean_rows_per_group >= 96.0 ? 0 : 1; }

int gemm_mx_tile_m() { return ShapeLargeMX::BM; }

template <class S>
hipError_t launch_mx_shape(const GemmCall& c, hipStream_t s) {
  if (c.c_codes) {
    // SwiGLU GEMM with an MXFP8 output (codes + block scales; N a multiple of 32)
    if (c.swiglu_h <= 0 || !c.gather || c.scatter || !c.c_scales || c.N % 32 != 0) return hipErrorInvalidValue;
    const int64_t ntn = (c.N + S::BN / 2 - 1) / (S::BN / 2);
    const int64_t upper = static_cast<int64_t>(c.tiles.cap) * ntn;
    if (upper <= 0 || c.rows_bound <= 0) return hipSuccess;
    int64_t grid = std::min<int64_t>(upper, static_cast<int64_t>(device_cu_count()) * S::WG_PER_CU);
    grid = ((grid + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL((gemm_bf16_kernel<S, true, true, false, false, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(S::NT), 0, s, c);
    return hipGetLastError();
  }
  return launch_shape<S>(c, s, S::WG_PER_CU);
}

hipError_t launch_gemm_mx(const GemmCall& c, hipStream_t s) {
  if (c.dense_M > 0 || c.Kd % ShapeLargeMX::BK != 0 || !c.a_scale || !c.b_scale) return hipErrorInvalidValue;
  // four k-stages of scales per 16-byte load: whole groups, 16-byte aligned rows
  const bool grouped = c.Kd % (4 * ShapeLargeMXG::BK) == 0 && c.a_scale_ld % 16 == 0 && c.b_scale_ld % 16 == 0 &&
                       c.b_scale_group_stride % 16 == 0 && reinterpret_cast<uintptr_t>(c.a_scale) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(c.b_scale) % 16 == 0;
  return grouped ? launch_mx_shape<ShapeLargeMXG>(c, s) : launch_mx_shape<ShapeLargeMX>(c, s);
}

hipError_t launch_gemm_bf16(const GemmCall& c, int variant, hipStream_t s) {
  if (variant == 0) return launch_shape<ShapeLarge>(c, s, ShapeLarge::WG_PER_CU);
  return launch_shape<ShapeSmall>(c, s, ShapeSmall::WG_PER_CU);
}

namespace {

// Input gradients: grouped rows like the forward, weights read contraction-major (W[e] as
// stored is (contraction, N)). Epilogue: SwiGLU backward, scatter, or plain rows.
template <class S>
hipError_t launch_dgrad_shape(const GemmCall& c, hipStream_t s) {
  const int64_t ntn = (c.N + S::BN - 1) / S::BN;
  const int64_t upper = static_cast<int64_t>(c.tiles.cap) * ntn;
  if (upper <= 0 || c.rows_bound <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(upper, static_cast<int64_t>(device_cu_count()) * S::WG_PER_CU);
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  const dim3 g(static_cast<unsigned>(grid)), b(S::NT);
  if (c.bwd_h > 0) {
    if (c.scatter || !c.h_in) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, false, false, false, 2, false, true>), g, b, 0, s, c);
  } else if (c.scatter) {
    hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, true, false, false, 2>), g, b, 0, s, c);
  } else {
    hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, false, false, false, 2>), g, b, 0, s, c);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_dgrad(const GemmCall& c, int variant, hipStream_t s) {
  if (c.trans != 2 || c.gather || c.swiglu_h > 0 || c.group_offsets || c.dense_M > 0 || c.N % 8 != 0)
    return hipErrorInvalidValue;
  if (variant == 0) return launch_dgrad_shape<ShapeLarge>(c, s);
  return launch_dgrad_shape<ShapeSmall>(c, s);
}

hipError_t launch_gemm_bf16_wgrad(const GemmCall& c, hipStream_t s) {
  using S = ShapeLarge;
  if (c.trans != 3 || !c.group_offsets || !c.tile_counter || c.gather || c.scatter || c.bwd_h > 0 ||
      c.swiglu_h > 0 ||
      c.dense_M <= 0 || c.groups <= 0 || c.N <= 0 || c.N % 8 != 0 || c.dense_M % 8 != 0)
    return hipErrorInvalidValue;
  const int64_t ntn = (c.N + S::BN - 1) / S::BN;
  const int64_t upper = static_cast<int64_t>(c.groups) * ((c.dense_M + S::BM - 1) / S::BM) * ntn;
  int64_t grid = std::min<int64_t>(upper, static_cast<int64_t>(device_cu_count()) * S::WG_PER_CU);
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, false, false, false, 3, true>), dim3(static_cast<unsigned>(grid)),
                     dim3(S::NT), 0, s, c);
  return hipGetLastError();
}

}  // namespace moe
