// Dense and 2:4-sparse GEMM kernels for gfx950 (one skeleton, four kinds).
//
// C[M][N] = A[M][K] . W[K][N].  The 2:4 kinds read W from its compressed
// form (two kept values per group of four along K plus 2-bit positions,
// GPUSQ-ViT "Boost Vision Transformer with GPU-Friendly Sparsity and
// Quantization", abstract) and feed the gfx950 sparse matrix instructions,
// whose sparse operand is the instruction's row operand.  W's sparsity runs
// along K inside an output column, so the kernels compute the transposed
// product C^T = W^T . A^T: instruction rows are output channels n (sparse
// operand: kept values of W^T row n), instruction columns are tokens m
// (dense operand: a row of A, K contiguous).  The hardware selects, per kept
// value, the matching activation by the 2-bit position; no software gather
// of A is needed.  The dense kinds run the same skeleton with the dense
// instruction so that the sparse-vs-dense comparison isolates the matrix
// instruction.
//
// Work decomposition
//   * workgroup = WM x WN waves (8 for the large tiles: two per SIMD); tile =
//     BM tokens x BN channels; every wave owns TM x TN 32x32 blocks
//     (BM = 32*WM*TM, BN = 32*WN*TN);
//   * K advances in stages of 128 bytes of an A row (f16: 64 k, i8: 128 k);
//     every stage is copied global -> LDS with direct-to-LDS loads (no
//     register staging) into a ring of STAGES buffers: stage s+STAGES is
//     fetched while stage s+1 is read into registers and stage s feeds the
//     matrix cores.  One explicit wait on the vector-memory counter plus one
//     barrier per stage hand a stage over;
//   * the sparse kinds' metadata either travels with each stage or, on the
//     tiles that use it, is fetched in blocks of several stages into a ring
//     of its own (fewer, longer row segments per load);
//   * on some tiles (SmallP, the sparse T64N) a second group of waves does
//     all the loading and the compute waves only read LDS and issue matrix
//     instructions; both groups meet at the same per-stage barrier;
//   * fragments are double-buffered in registers: the LDS reads of the next
//     k-step are issued between the matrix instructions of the current one
//     (scheduling hints interleave them), so one wave per SIMD keeps its
//     matrix pipe busy without waiting on LDS latency;
//   * LDS rows are XOR-swizzled in 16-byte chunks so that the rows read by one
//     fragment load fall into distinct banks; the direct-to-LDS lane order is
//     fixed (lane i writes bytes 16i..16i+15 of the wave's 1 KiB), so each lane
//     fetches the global chunk that belongs at its swizzled position;
//   * block ids are remapped so each XCD works on a contiguous range of tiles
//     (grouped GM tile-rows at a time), which keeps shared A rows and W
//     columns in that XCD's L2;
//   * epilogue: the accumulators go through LDS as row-major [token][channel]
//     slabs, so C is written as whole contiguous row segments, 16 bytes per
//     lane (fp16 kinds: fp16 rounded to nearest even; int8 kinds: raw int32,
//     or y = float(acc) * scale[n] (+ bias[n]) written as fp32, as fp16
//     rounded to nearest even, or as int8 rounded to nearest even and
//     saturated to [-128, 127]);
//   * a tile starts its K loop at stage 0 or, for the sparse 128 x 128 and
//     64 x 128 tiles, at a stage rotated by its tile id (measured per tile
//     shape, see ROT);
//   * split K (gridDim.y > 1, EPI_PART): workgroup (tile, y) runs K-stage range
//     y and writes its raw accumulators to slice y of a workspace, which
//     splitk.hip sums and finishes with the kind's epilogue.
//
// Instruction operand layouts (64-lane wave, h = lane / 32, r = lane % 32):
//   dense f16 32x32x16 : row-op lane holds k = 8h .. 8h+7 of its row r
//   dense i8  32x32x32 : k = 16h .. 16h+15
//   sparse f16 32x32x32: sparse row-op lane holds the 8 kept values of row r
//                        for k in [16h, 16h+16) (4 groups, ascending), slot c's
//                        two-bit position at bits 2c of the index operand; the
//                        dense column-op lane holds, as elements 0..7 and
//                        8..15, k = 8h .. 8h+7 and k = 16+8h .. 16+8h+7 of
//                        column r (measured on gfx950 with one-wave probes)
//   sparse i8 32x32x64 : sparse lane: 16 kept values for k in [32h, 32h+32),
//                        16 positions = 32 index bits; dense lane: elements
//                        0..15 = k 16h .., elements 16..31 = k 32+16h ..
//   accumulator        : lane holds rows 8*(i/4) + 4h + i%4 (i = 0..15) of
//                        column r
// The compressed pack stores slot j's position at bits 2*(j%16) of word j/16,
// which is exactly the index operand for these ranges, so meta words are fed
// to the instruction as stored (shifted by 16 bits for the upper f16 half).
#include "common.h"
#include "launch.h"

namespace ssg {

enum Kind { DENSE_F16 = 0, W24_F16 = 1, DENSE_I8 = 2, W24_I8 = 3 };
// EPI_F16: fp16 kinds.  int8 kinds: EPI_I32 raw accumulators; the others
// compute y = float(acc) * scale[n] (+ bias[n]), each step rounded to nearest
// even, then store y as fp32, fp16 or saturated int8.  EPI_PART (split K, any
// kind): the raw accumulators (fp32 or int32) of K-split blockIdx.y go to its
// [M][N] slice of the workspace passed as C; a second kernel sums the slices.
enum Epi { EPI_F16 = 0, EPI_I32 = 1, EPI_F32_SCALE = 2, EPI_F16_SCALE = 3, EPI_I8_SCALE = 4, EPI_PART = 5 };

template <int KIND>
struct KindTraits;

template <>
struct KindTraits<DENSE_F16> {
    static constexpr bool kSparse = false, kI8 = false;
    static constexpr int kWB = 128;  // W bytes per row per stage
    static constexpr int kMW = 0;    // meta words per row per stage
    static constexpr int kNI = 4;    // instructions per stage
};
template <>
struct KindTraits<W24_F16> {
    static constexpr bool kSparse = true, kI8 = false;
    static constexpr int kWB = 64, kMW = 2, kNI = 2;
};
template <>
struct KindTraits<DENSE_I8> {
    static constexpr bool kSparse = false, kI8 = true;
    static constexpr int kWB = 128, kMW = 0, kNI = 4;
};
template <>
struct KindTraits<W24_I8> {
    static constexpr bool kSparse = true, kI8 = true;
    static constexpr int kWB = 64, kMW = 4, kNI = 2;
};

// 16-byte chunk swizzles (see header comment).
__device__ __forceinline__ int swz128(int row, int col) { return col ^ ((row ^ (row >> 3)) & 7); }
__device__ __forceinline__ int swz256(int row, int col) { return col ^ (row & 15); }
__device__ __forceinline__ int swz64(int row, int col) { return col ^ (((row >> 1) ^ (row >> 3)) & 3); }
// swizzle of a row of RB bytes (64, 128 or 256)
template <int RB>
__device__ __forceinline__ int swzw(int row, int col) {
    if constexpr (RB == 64) return swz64(row, col);
    else if constexpr (RB == 128) return swz128(row, col);
    else return swz256(row, col);
}

template <int KIND>
struct AccOf {
    using T = typename std::conditional<KindTraits<KIND>::kI8, intx16, floatx16>::type;
};

__device__ __forceinline__ u32x4 lds16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Direct-to-LDS loads through a buffer resource: lane i of the wave reads
// 16 (4) bytes at byte offset `off` of the buffer and writes them to
// wave_base + 16*i (4*i); wave_base must be uniform across the wave.  The
// buffer form moves a few per cent more per wave than the flat-address form
// (L2 → LDS microbenchmark on MI355X), and reads past the buffer's size
// return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t *wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)wave_base, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t *wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)wave_base, 4, off, 0, 0, 0);
}

// Waits until at most N vector-memory operations of this wave are
// outstanding, then synchronises the workgroup (no memory fence: LDS data
// here is produced by direct-to-LDS loads, which the counter tracks).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Same, after this wave's LDS reads have completed as well.
template <int N>
__device__ __forceinline__ void wait_lgkm_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// One matrix instruction.  w: the row operand (kept W^T values, or dense W^T
// for the dense kinds); a: the column operand (activations).  For the sparse
// kinds a holds 32 bytes; the dense kinds use its low 16 bytes.
template <int KIND>
__device__ __forceinline__ void mma(typename AccOf<KIND>::T &acc, u32x4 w, u32x8 a, uint32_t idx) {
    if constexpr (KIND == W24_F16) {
        acc = __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(half8, w), __builtin_bit_cast(half16, a),
                                                        acc, int(idx), 0, 0);
    } else if constexpr (KIND == W24_I8) {
        acc = __builtin_amdgcn_smfmac_i32_32x32x64_i8(__builtin_bit_cast(intx4, w), __builtin_bit_cast(intx8, a), acc,
                                                       int(idx), 0, 0);
    } else if constexpr (KIND == DENSE_F16) {
        const u32x4 lo = __builtin_shufflevector(a, a, 0, 1, 2, 3);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, w), __builtin_bit_cast(half8, lo), acc,
                                                      0, 0, 0);
    } else {
        const u32x4 lo = __builtin_shufflevector(a, a, 0, 1, 2, 3);
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(intx4, w), __builtin_bit_cast(intx4, lo), acc,
                                                     0, 0, 0);
    }
}

// Epilogue store of one 16-byte piece; nontemporal stores stream past L2.
template <bool NTS>
__device__ __forceinline__ void store16(void *p, u32x4 v) {
    if constexpr (NTS) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
    else *reinterpret_cast<u32x4 *>(p) = v;
}

// Tile configuration: WM x WN waves, TM x TN 32x32 blocks per wave, STAGES
// LDS stage buffers (prefetch distance), GM tile-rows per L2 group,
// nontemporal C stores, ROT: each tile starts its K loop at its own stage.
// By default every wave issues an equal share of each stage's direct-to-LDS
// loads.
// MP: K stages per metadata block of the sparse kinds (0: each stage's
// metadata travels with the stage).  PROD: the workgroup has as many
// loader waves as compute waves; the loader waves issue every direct-to-LDS
// load and the compute waves only read LDS and run the matrix instructions.
// NLD (without PROD): only compute waves 0..NLD-1 issue the loads (0: all).
// DK: K depth of a stage in units of 128 bytes of an A row.
template <int WM_, int WN_, int TM_, int TN_, int STAGES_, int GM_, bool NTS_, bool ROT_, int MP_ = 0,
          bool PROD_ = false, int NLD_ = 0, int DK_ = 1>
struct Cfg {
    static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_, STAGES = STAGES_, GM = GM_;
    static constexpr bool NTS = NTS_, ROT = ROT_, PROD = PROD_;
    static constexpr int MP = MP_, NLD = NLD_, DK = DK_;
};

template <int KIND, class CF>
struct Layout {
    using KT = KindTraits<KIND>;
    static constexpr int NW = CF::WM * CF::WN;           // compute waves (and loader waves)
    static constexpr int NT = NW * kWave * (CF::PROD ? 2 : 1);  // threads
    static constexpr int BM = CF::WM * CF::TM * 32;
    static constexpr int BN = CF::WN * CF::TN * 32;
    static constexpr int DK = CF::DK;
    static constexpr int AB = 128 * DK;      // A bytes per row per stage
    static constexpr int NI = KT::kNI * DK;  // matrix instructions (k-steps) per stage
    static constexpr int WB = KT::kWB * DK;
    static constexpr int MW = KT::kMW * DK;
    static constexpr int A_STAGE = BM * AB;
    static constexpr int W_STAGE = BN * WB;
    static constexpr int M_BYTES = BN * MW * 4;  // metadata bytes of one stage
    // Metadata blocks (MP > 0): the metadata of MP consecutive stages sits
    // in one block of its own ring instead of in the stage buffers, stored
    // row-major [BN][MP * MW] words, so that every 256-byte load covers
    // MP * MW * 4 contiguous bytes of a row (8 rows) rather than 8 or 16
    // bytes of 32 or 16 rows: the loads touch MP times fewer cache lines.
    // A block is fetched in MP parts, one with each of the MP stage loads
    // before its first stage; MSLOTS blocks are kept so that a part never
    // overwrites a block that a stage still in the ring reads.
    static constexpr int MP = KT::kSparse ? CF::MP : 0;
    static constexpr int M_STAGE = MP ? 0 : M_BYTES;
    static constexpr int STAGE = A_STAGE + W_STAGE + M_STAGE;
    static constexpr int RW = MP * MW;  // words per row in a block
    static constexpr int MBLK = MP * M_BYTES;
    static constexpr int MSLOTS = MP ? 2 + (CF::STAGES - 2 + MP - 1) / MP : 0;
    static constexpr int MRING = MSLOTS * MBLK;
    static_assert(MP == 0 || (64 % RW == 0 && BN % MP == 0), "metadata block shape");
    // direct-to-LDS instructions per wave per stage (each moves 1 KiB, or
    // 256 bytes for the 4-byte meta loads).  A 64-channel fp16 tile has 2
    // meta chunks of 256 bytes for 4 waves: then waves w and w + MCH load the
    // same chunk into the same LDS bytes (identical data), so that every wave
    // issues the same number of loads per stage and one counter value means
    // "stage complete" for all of them.
    static constexpr int MCH = M_BYTES / 256;
    // waves that issue the loads (the loader group, or the first NLD compute waves)
    static constexpr int NL = CF::PROD || CF::NLD == 0 ? NW : CF::NLD;
    static constexpr int LA = A_STAGE / 1024 / NL;
    static constexpr int LW = W_STAGE / 1024 / NL;
    static constexpr int LM = MCH >= NL ? MCH / NL : (MCH > 0 ? 1 : 0);
    static constexpr int L = LA + LW + LM;
    static_assert(LA * NL * 1024 == A_STAGE && LW * NL * 1024 == W_STAGE && MCH * 256 == M_BYTES &&
                      (MCH == 0 || MCH % NL == 0 || NL % MCH == 0),
                  "stage does not split evenly over the waves");
    // meta chunk of this wave's j-th meta load (no modulo unless chunks are
    // shared: on the 128 x 256 int8 tiles it cost the registers that keep
    // two workgroups per CU)
    static __device__ __forceinline__ int mchunk(int j, int wave) {
        if constexpr (MCH >= NL) return j * NL + wave;
        else return wave % (MCH > 0 ? MCH : 1);
    }
    // word position of (row, w) inside a metadata block: XOR-swizzled so that
    // the 32 rows of one fragment read fall into distinct banks
    static __device__ __forceinline__ int mword(int row, int w) {
        return row * RW + (w ^ ((row * RW / 32) & (RW - 1)));
    }
};

template <int KIND, int EPI, class CF>
__global__ void __launch_bounds__(CF::WM *CF::WN * 64 * (CF::PROD ? 2 : 1))
gemm_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ Wv, const uint32_t *__restrict__ meta,
            const float *__restrict__ scale, const float *__restrict__ bias, void *__restrict__ C, int M, int N,
            int K, int stages) {
    using KT = KindTraits<KIND>;
    using LY = Layout<KIND, CF>;
    using Acc = typename AccOf<KIND>::T;
    constexpr int TM = CF::TM, TN = CF::TN, GM = CF::GM, NB = CF::STAGES;
    constexpr int WM = CF::WM;
    constexpr int BM = LY::BM, BN = LY::BN, WB = LY::WB, MW = LY::MW;
    constexpr int A_STAGE = LY::A_STAGE, W_STAGE = LY::W_STAGE, STAGE = LY::STAGE;
    constexpr int SA = KT::kI8 ? 1 : 2;  // bytes per element
    // LDS-staged epilogue: each wave owns 32 token rows x TN*32 channels per pass
    constexpr int OB = (EPI == EPI_F16 || EPI == EPI_F16_SCALE) ? 2 : (EPI == EPI_I8_SCALE ? 1 : 4);  // output bytes
    constexpr int EROW = TN * 32 * OB + 16;       // padded LDS row (odd multiple of 16 B)
    constexpr int EWAVE = 32 * EROW;
    constexpr int EPASS = (TM * EWAVE * LY::NW <= CF::STAGES * STAGE) ? TM : 1;
    constexpr int SMEM_EPI = EPASS * EWAVE * LY::NW;
    constexpr int SMEM_MAIN = CF::STAGES * STAGE + LY::MRING;
    constexpr int SMEM = (SMEM_MAIN > SMEM_EPI) ? SMEM_MAIN : SMEM_EPI;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // With loader waves (PROD), waves NW.. load and waves 0..NW-1 compute;
    // `wave` is a wave's index within its group.
    constexpr bool PROD = CF::PROD;
    const bool loader = PROD && (tid >> 6) >= LY::NW;
    const int wave = loader ? (tid >> 6) - LY::NW : tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int h = lane >> 5, r = lane & 31;

    // ---- tile assignment: XCD-contiguous ranges, GM tile-rows per group
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int b = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int group = b / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_group = b % (GM * tiles_n);
    const int tile_m = first_m + in_group % gm;
    const int tile_n = in_group / gm;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int64_t a_row = int64_t(K) * SA;                  // bytes per A row
    const int64_t w_row = KT::kSparse ? a_row / 2 : a_row;  // bytes per W row
    const int64_t m_row = K / 32;                            // meta words per row
    // S = K stages of this workgroup (128 bytes of an A row each): all of them,
    // or, with K split over gridDim.y, split blockIdx.y's equal share.  The
    // mask is a value-range hint (the host's 4 GiB operand limit keeps S below
    // 2^19): with S known to be small the compiler keeps the stage address
    // arithmetic narrow, which holds the 128 x 256 tiles within the 256
    // registers that two workgroups per CU allow (260 without it).
    const int S = stages & 0xffffff;
    const int ks0 = int(blockIdx.y) * S;

    // ---- direct-to-LDS sources: instruction j of this wave fills the wave's
    // j-th KiB of the A (or W) stage; lane -> (row, position) -> global chunk.
    // (32-bit byte offsets from the uniform base pointers keep the per-lane
    // address state small.)
    uint32_t oa[LY::LA];
#pragma unroll
    for (int j = 0; j < LY::LA; ++j) {
        const int byte = (j * LY::NL + wave) * 1024 + lane * 16;
        const int row = byte / LY::AB, pos = (byte / 16) % (LY::AB / 16);
        oa[j] = uint32_t(min(m0 + row, M - 1)) * uint32_t(a_row) + swzw<LY::AB>(row, pos) * 16;
    }
    uint32_t ow[LY::LW];
#pragma unroll
    for (int j = 0; j < LY::LW; ++j) {
        const int byte = (j * LY::NL + wave) * 1024 + lane * 16;
        const int row = byte / WB, pos = (byte / 16) % (WB / 16);
        ow[j] = uint32_t(min(n0 + row, N - 1)) * uint32_t(w_row) + swzw<WB>(row, pos) * 16;
    }
    uint32_t om[LY::LM > 0 ? LY::LM : 1];
#pragma unroll
    for (int j = 0; j < LY::LM; ++j) {
        const int word = LY::mchunk(j, wave) * 64 + lane;  // row-major [BN][MW]
        const int row = word / (MW > 0 ? MW : 1), w = word % (MW > 0 ? MW : 1);
        om[j] = (uint32_t(min(n0 + row, N - 1)) * uint32_t(m_row) + w) * 4;
    }
    constexpr int RW = LY::MP ? LY::RW : 1;
    const uint8_t *meta_b = reinterpret_cast<const uint8_t *>(meta);

    // Where a tile starts its K loop.  From stage 0, the tiles in flight on an
    // XCD read the same K slice at about the same time, so one L2 fill serves
    // several of them; rotated (tile b starts at stage b mod S), they read
    // different slices, which spreads their requests over more memory
    // channels but gives up that sharing.  The K reduction may run in any
    // order, and the order is fixed per tile, so results stay deterministic
    // either way.  Which one is faster was measured per tile shape on MI355X
    // (ROT in the tile configurations below).
    const int rot = CF::ROT ? b % S : 0;
    // (the host caps A and W below 4 GiB, so every byte count fits 32 bits)
    const __amdgpu_buffer_rsrc_t bufA = buffer_of(A, uint32_t(int64_t(M) * a_row));
    const __amdgpu_buffer_rsrc_t bufW = buffer_of(Wv, uint32_t(int64_t(N) * w_row));
    const __amdgpu_buffer_rsrc_t bufM = buffer_of(meta_b, KT::kSparse ? uint32_t(int64_t(N) * m_row * 4) : 0u);
    // Part t - (c - 1) * MP - 1 of metadata block c = ceil(t / MP), loaded
    // with the loads of stage t (t < 0: the prologue's parts of block 0).
    // Each part is MCH 256-byte chunks, BN / MP rows.  Lane's word is (row,
    // stored position p) of the block; it holds word w = p ^ swizzle of the
    // row's metadata for block stage q = w / MW, i.e. local stage c * MP + q
    // (past the last stage: any valid word, never read).
    auto issue_meta = [&](int t) {
        if constexpr (LY::MP > 0) {
            constexpr int MPr = LY::MP > 0 ? LY::MP : 1;
            const int c = (t + MPr - 1) / MPr;  // ceil(t / MP); t + MP - 1 >= 0
            const int part = t - (c * MPr - MPr + 1);
            uint8_t *blk = smem + NB * STAGE + (c % LY::MSLOTS) * LY::MBLK;
#pragma unroll
            for (int j = 0; j < LY::LM; ++j) {
                const int row = (part * LY::MCH + LY::mchunk(j, wave)) * (64 / RW) + lane / RW;
                const int w = (lane % RW) ^ ((row * RW / 32) & (RW - 1));
                const int sl = min(c * MPr + w / MW, S - 1);
                const int sg = ks0 + ((sl + rot < S) ? sl + rot : sl + rot - S);
                const uint32_t off =
                    (uint32_t(min(n0 + row, N - 1)) * uint32_t(m_row) + uint32_t(sg * MW + w % MW)) * 4;
                dma4(bufM, off, blk + (part * LY::MCH + LY::mchunk(j, wave)) * 256);
            }
        }
    };
    const bool issuer = LY::NL == LY::NW || wave < LY::NL;  // (with PROD: the loaders)
    auto issue = [&](int s) {
        if (!issuer) return;
        uint8_t *base = smem + (s % NB) * STAGE;
        const int sg = ks0 + ((s + rot < S) ? s + rot : s + rot - S);  // global K stage
#pragma unroll
        for (int j = 0; j < LY::LA; ++j)
            dma16(bufA, oa[j] + uint32_t(sg * LY::AB), base + (j * LY::NL + wave) * 1024);
#pragma unroll
        for (int j = 0; j < LY::LW; ++j)
            dma16(bufW, ow[j] + uint32_t(sg * WB), base + A_STAGE + (j * LY::NL + wave) * 1024);
        if constexpr (LY::MP == 0) {
#pragma unroll
            for (int j = 0; j < LY::LM; ++j)
                dma4(bufM, om[j] + uint32_t(sg * MW * 4), base + A_STAGE + W_STAGE + LY::mchunk(j, wave) * 256);
        } else {
            issue_meta(s);
        }
    };

    // Fragments of one k-step (one matrix instruction deep) for the wave's
    // TN channel blocks and TM token blocks.
    struct Frag {
        u32x4 w[TN];
        uint32_t idx[TN];
        u32x8 a[TM];
    };
    auto load_frag = [&](int s, int kk, Frag &F) {
        const uint8_t *bA = smem + (s % NB) * STAGE;
        const uint8_t *bW = bA + A_STAGE;
        const uint32_t *bM = reinterpret_cast<const uint32_t *>(bA + A_STAGE + W_STAGE);
        constexpr int MPr = LY::MP > 0 ? LY::MP : 1;
        const uint32_t *bB =
            reinterpret_cast<const uint32_t *>(smem + NB * STAGE + ((s / MPr) % (LY::MP ? LY::MSLOTS : 1)) * LY::MBLK);
        const int q = (s % MPr) * MW;  // first word of stage s in a block row
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int row = wn * TN * 32 + tn * 32 + r;
            F.w[tn] = lds16(bW + row * WB + swzw<WB>(row, 2 * kk + h) * 16);
            if constexpr (LY::MP > 0 && KIND == W24_F16) F.idx[tn] = bB[LY::mword(row, q + kk)] >> (16 * h);
            else if constexpr (LY::MP > 0 && KIND == W24_I8) F.idx[tn] = bB[LY::mword(row, q + 2 * kk + h)];
            else if constexpr (KIND == W24_F16) F.idx[tn] = bM[row * MW + kk] >> (16 * h);
            else if constexpr (KIND == W24_I8) F.idx[tn] = bM[row * MW + 2 * kk + h];
            else F.idx[tn] = 0;
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int row = wm * TM * 32 + tm * 32 + r;
            if constexpr (KT::kSparse) {
                // two 16-byte pieces of the 64-byte window: bytes 16h.. and 32+16h..
                const u32x4 lo = lds16(bA + row * LY::AB + swzw<LY::AB>(row, 4 * kk + h) * 16);
                const u32x4 hi = lds16(bA + row * LY::AB + swzw<LY::AB>(row, 4 * kk + 2 + h) * 16);
                F.a[tm] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                const u32x4 lo = lds16(bA + row * LY::AB + swzw<LY::AB>(row, 2 * kk + h) * 16);
                F.a[tm] = __builtin_shufflevector(lo, lo, 0, 1, 2, 3, 0, 1, 2, 3);
            }
        }
    };

    Acc acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = Acc{};

    auto mma_frag = [&](const Frag &F) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) mma<KIND>(acc[tn][tm], F.w[tn], F.a[tm], F.idx[tn]);
    };
    // Interleave hint: one matrix instruction, then its share of LDS reads.
    constexpr int NMMA = TN * TM;
    constexpr int NRD = TN * (KT::kSparse ? 2 : 1) + TM * (KT::kSparse ? 2 : 1);
    constexpr int RPM = (NRD + NMMA - 1) / NMMA;
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NMMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // matrix
            __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);  // LDS reads
        }
    };

    // Pipeline: NB stage buffers, the stage s+NB is fetched while stage s+1 is
    // read into registers and stage s feeds the matrix cores.  Within a stage
    // the next k-step's fragments are read during the current k-step's
    // instructions; the stage hand-off (wait + barrier) sits before the last
    // k-step's instructions so that the next stage's first fragments overlap
    // them too.
    if (!PROD || loader) {
        if constexpr (LY::MP > 1)
            for (int t = 1 - LY::MP; t < 0; ++t) issue_meta(t);
#pragma unroll
        for (int s = 0; s < NB; ++s)
            if (s < S) issue(s);
    }
    if (NB < S) wait_vm_barrier<(NB - 1) * LY::L>();
    else wait_vm_barrier<0>();
    if (loader) {
        // the same barriers as the compute waves' stages: after the one that
        // ends stage s, stage s's buffer is free for stage s + NB
        int s = 0;
        for (; s + NB < S; ++s) {
            wait_vm_barrier<(NB - 2) * LY::L>();
            issue(s + NB);
        }
        for (; s < S; ++s) wait_vm_barrier<0>();
    } else {
        Frag F[2];
        load_frag(0, 0, F[0]);

        // One stage; STEADY: the ring still has a stage to fetch (s + NB < S).
        // The next stage's first fragments are read unconditionally: on the last
        // stage this reads a valid, stale buffer whose values are never used.
        auto stage = [&](int s, auto steady) {
#pragma unroll
            for (int kk = 0; kk < LY::NI; ++kk) {
                Frag &cur = F[kk & 1];
                Frag &nxt = F[(kk + 1) & 1];
                if (kk + 1 < LY::NI) {
                    load_frag(s, kk + 1, nxt);
                } else {
                    // stage s is fully in registers; stage s+1 must be complete
                    if constexpr (decltype(steady)::value) {
                        wait_lgkm_vm_barrier<(NB - 2) * LY::L>();
                        if constexpr (!PROD) issue(s + NB);  // reuses stage s's buffer
                    } else {
                        wait_lgkm_vm_barrier<0>();
                    }
                    load_frag(s + 1, 0, nxt);
                }
                mma_frag(cur);
                interleave();
            }
        };
        int s = 0;
        for (; s + NB < S; ++s) stage(s, std::true_type{});
        for (; s < S; ++s) stage(s, std::false_type{});
    }

    // ---- epilogue.  Lane (h, r) holds, for 32x32 block (tn, tm) and q = 0..3,
    // channels n = tn*32 + 8q + 4h .. +3 of token m = tm*32 + r.
    auto convert = [&](const Acc &v, int q, int n) -> u32x4 {
        u32x4 o = u32x4{0, 0, 0, 0};
        if constexpr (EPI == EPI_F16) {
            o.x = pack_half2_rne(v[4 * q + 0], v[4 * q + 1]);
            o.y = pack_half2_rne(v[4 * q + 2], v[4 * q + 3]);
        } else if constexpr (EPI == EPI_PART) {
            // (whole 4-vectors are bit-cast: a bit-cast of a single element of
            // the 16-wide accumulator vector yielded element 0 for every lane)
            using E4 = typename std::conditional<KT::kI8, intx4, floatx4>::type;
            const E4 t = E4{v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            o = __builtin_bit_cast(u32x4, t);
        } else if constexpr (EPI == EPI_I32) {
            o.x = uint32_t(v[4 * q + 0]);
            o.y = uint32_t(v[4 * q + 1]);
            o.z = uint32_t(v[4 * q + 2]);
            o.w = uint32_t(v[4 * q + 3]);
        } else {
            const int nc = min(n, N - 4);
            const floatx4 sc = *reinterpret_cast<const floatx4 *>(scale + nc);
            floatx4 f;
            f.x = __fmul_rn(float(v[4 * q + 0]), sc.x);
            f.y = __fmul_rn(float(v[4 * q + 1]), sc.y);
            f.z = __fmul_rn(float(v[4 * q + 2]), sc.z);
            f.w = __fmul_rn(float(v[4 * q + 3]), sc.w);
            if (bias) {
                const floatx4 bi = *reinterpret_cast<const floatx4 *>(bias + nc);
                f.x = __fadd_rn(f.x, bi.x);
                f.y = __fadd_rn(f.y, bi.y);
                f.z = __fadd_rn(f.z, bi.z);
                f.w = __fadd_rn(f.w, bi.w);
            }
            if constexpr (EPI == EPI_F32_SCALE) {
                o = __builtin_bit_cast(u32x4, f);
            } else if constexpr (EPI == EPI_F16_SCALE) {
                o.x = pack_half2_rne(f.x, f.y);
                o.y = pack_half2_rne(f.z, f.w);
            } else {
                // round to nearest even, saturate, pack four int8 into one word
                auto q8 = [](float y) -> uint32_t {
                    const float r = fminf(fmaxf(__builtin_rintf(y), -128.0f), 127.0f);
                    return uint32_t(int32_t(r)) & 0xffu;
                };
                o.x = q8(f.x) | (q8(f.y) << 8) | (q8(f.z) << 16) | (q8(f.w) << 24);
            }
        }
        return o;
    };

    // Stage 32-token slabs of the wave's accumulators through LDS as
    // row-major [token][channel], then store whole row segments
    // (TN*32*OB contiguous bytes per token) with 16 bytes per lane.
    constexpr int CPR = TN * 32 * OB / 16;  // 16-byte chunks per token row
    constexpr int RPI = kWave / CPR;        // token rows per store instruction
    static_assert(RPI * CPR == kWave, "row segment must tile a wave");
    __syncthreads();  // every wave is done reading the stage buffers
    uint8_t *const Cb = reinterpret_cast<uint8_t *>(C) + (EPI == EPI_PART ? int64_t(blockIdx.y) * M * N * OB : 0);
    uint8_t *ew = smem + wave * EPASS * EWAVE;  // (compute waves)
    const int nw = n0 + wn * TN * 32;  // first channel of the wave
#pragma unroll
    for (int tp = 0; tp < TM; tp += EPASS) {
        if (!loader) {
#pragma unroll
            for (int e = 0; e < EPASS; ++e) {
                uint8_t *slab = ew + e * EWAVE + r * EROW;
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int c = tn * 32 + q * 8 + h * 4;
                        const u32x4 o = convert(acc[tn][tp + e], q, nw + c);
                        if constexpr (OB == 1) *reinterpret_cast<uint32_t *>(slab + c) = o.x;
                        else if constexpr (OB == 2) *reinterpret_cast<u32x2 *>(slab + c * 2) = u32x2{o.x, o.y};
                        else *reinterpret_cast<u32x4 *>(slab + c * 4) = o;
                    }
            }
        }
        __syncthreads();
        if (!loader) {
#pragma unroll
            for (int e = 0; e < EPASS; ++e) {
#pragma unroll
                for (int i = 0; i < 32 / RPI; ++i) {
                    const int row = i * RPI + lane / CPR, ch = lane % CPR;
                    const int m = m0 + wm * TM * 32 + (tp + e) * 32 + row;
                    const int n = nw + ch * (16 / OB);
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(ew + e * EWAVE + row * EROW + ch * 16);
                    if (m < M && n < N) store16<CF::NTS>(Cb + (int64_t(m) * N + n) * OB, v);
                }
            }
        }
        if (tp + EPASS < TM) __syncthreads();
    }
}

template <int KIND, int EPI, class CF>
static hipError_t launch(const void *A, const void *Wv, const uint32_t *meta, const float *scale,
                         const float *bias, void *C, int M, int N, int K, hipStream_t st, int splits = 1) {
    using LY = Layout<KIND, CF>;
    const int nb = ((M + LY::BM - 1) / LY::BM) * ((N + LY::BN - 1) / LY::BN);
    const int stages = K * (KindTraits<KIND>::kI8 ? 1 : 2) / (128 * CF::DK) / splits;
    hipLaunchKernelGGL((gemm_kernel<KIND, EPI, CF>), dim3(nb, splits), dim3(LY::NT), 0, st,
                       static_cast<const uint8_t *>(A), static_cast<const uint8_t *>(Wv), meta, scale, bias, C, M, N,
                       K, stages);
    return hipGetLastError();
}

// Tile shapes (measured on MI355X at the ViT / BERT / ViT-Base shapes):
//   Big    256 x 256, 8 waves of 64 tokens x 128 channels, one workgroup per
//          CU -- best once there are about as many tiles as CUs and K is long
//          enough to amortise the prologue.  On the fp16 2:4 tile and the
//          dense tiles only waves 0..3 issue the loads, so each SIMD keeps
//          one wave whose matrix work no load waits behind (fp16 2:4 ViT-L
//          qkv 27.5 -> 26.3 us, fc1 31.5 -> 30.8; dense fp16 28.9 -> 28.1
//          and 37.3 -> 36.2; with two of the eight waves loading, no gain;
//          the int8 2:4 tile would spill, and the int8 Small2 tile with two
//          of four waves loading ran the headline 46.0 -> 48.7 us);
//   Mid    128 x 256, 4 waves, 2 stages (two workgroups per CU) -- short-K
//          int8 GEMMs with one to two such tiles per CU;
//   Small  128 x 128, 4 waves, 3 stages (two workgroups per CU) -- long-K
//          int8 GEMMs with more than 256 (dense: 576) such tiles, and the
//          8-way K splits of few-tile fp16 GEMMs;
//   SmallP the same tile with 4 more waves that only load (one workgroup
//          per CU) and, for the sparse kinds, metadata blocks of 4 (fp16) or
//          2 (int8) stages -- narrow outputs (N = 1024) that would leave CUs
//          idle with big tiles: every fp16 GEMM without enough Big tiles
//          (other than the few-tile ones of T64 / T32 below), and the long-K
//          int8 ones up to 256 tiles (dense: 576).  Against Small,
//          graph-timed on cold input sets: fp16 2:4 4096 x 1024 x 4096
//          (M x N x K) 42.3 -> 38.9 us, 4096 x 768 x 3072 31.5 -> 28.4,
//          6144 x 1024 x 4096 (384 tiles) 67.6 -> 63.4, 6144 x 1536 x 4096
//          (576) 96.8 -> 87.0; dense fp16 4096 x 1024 x 4096 43.1 -> 41.5;
//          int8 2:4 4096 x 768 x 3072 17.5 -> 16.5 us, but 6144 x 1024 x
//          4096 37.0 -> 39.0.  The int8 2:4 tile (unsplit, K a multiple of
//          256) takes stages twice as deep in K, 256 k with the metadata in
//          the stage (int8 2:4 4096 x 1024 x 4096 23.5 -> 20.8 us, 4096 x
//          768 x 3072 16.6 -> 16.0, 3072 x 1024 x 4096 20.7 -> 19.8); the
//          fp16 tiles run slower so (4096 x 1024 x 4096 37.7 -> 43.6), and
//          the dense ones, with two such stages, too.  Neither part pays alone (fp16 2:4 4096 x 1024
//          x 4096: metadata blocks 46.6-46.9 us, loader waves 45-46, both
//          41.5, Small 44.7-45.2 in that session): the metadata blocks cut
//          the cache lines the loads touch (a copy of the kernel without
//          fragment reads and matrix instructions ran 40.1 -> 34.8 us), and
//          only with the loads moved off the compute waves does the full
//          kernel follow;
//   Small2 128 x 128, 4 waves, 2 stages (three int8 workgroups per CU) --
//          short-K int8 GEMMs whose Mid tiles would fill the chip more than
//          twice or less than once, and the dense int8 GEMMs at short K;
//   T64    64 x 64 and T64N 64 x 128, 4 waves of 32 x 32 / 32 x 64, 3 stages
//          (the sparse fp16 T64N with 4 loader waves and 4-stage metadata
//          blocks: 512 x 3072 x 1024 9.6 -> 9.1 us, 512 x 4096 x 1024
//          10.6 -> 10.0, 2048 x 1024 x 4096 32.0 -> 27.7; the dense one runs
//          slower so, 10.4 -> 11.0 us at 512 x 3072 x 1024)
//          -- GEMMs with at most 128 tiles of 128 x 128 (half the CUs; int8
//          with K <= 1024: 192), e.g. one GPU's share of a token-sharded
//          layer (M = 512).  With so few
//          tiles each workgroup's K loop runs alone on its CU, limited by
//          what its four waves can pull into LDS per stage; smaller tiles
//          put more CUs to work and each moves less (int8 2:4 512 x 1024 x
//          1024: 9.2 us on 128 x 128, 5.8 on 64 x 64; 512 x 4096 x 1024:
//          19.6 -> 12.6 us; fp16 2:4 512 x 1024 x 1024: 10.7 us -> 9.0 on
//          64 x 128).  A deeper ring (4-6 stages) on 128 x 128 gained nothing
//          there.  The fp16 kinds keep 64 x 128 once 64 x 64 tiles would
//          outnumber the CUs (dense fp16 512 x 1024 x 3072: 10.1 us on
//          64 x 128, 11.1 on 64 x 64); int8, with half as many K stages,
//          takes 64 x 64 throughout;
//   T32    32 x 32, one wave, 4 stages -- the smallest GEMMs (at most 512
//          such tiles and fewer than 64 K stages).  Against 64-row tiles in
//          one sweep (its first, 3-stage rotated form): fp16 2:4 256 x 512 x
//          512 5.2 -> 4.4 us, 384 x 1024 x 1024 7.3 -> 6.4; int8 2:4 128 x
//          4096 x 4096 12.3 -> 10.5; at 1024 tiles (1024 x 1024 outputs) the
//          64-row tiles are ahead again.  The 4-stage ring from stage 0
//          (ROT below) took 256 x 512 x 512 to 3.8 us.
// K-loop start (ROT), measured with both variants timed in one process over
// alternating rounds, on input sets rotated through more than twice the
// 256 MB Infinity Cache: every dense kind and the sparse Big and Mid tiles run
// 3-10 % faster from stage 0 (ViT-L qkv / fc1 / fc2, 4096x8192x1024,
// 4096x2048x4096), while the sparse 128 x 128 tiles run 4-10 % faster rotated
// (fp16 ViT-L fc2 42.1 vs 46.2 us, int8 4096x8192x1024 43.7 vs 47.7 us; the
// short-K int8 one is within noise either way).  So ROT = sparse kind on a
// 128 x 128 tile, and on the sparse 64 x 128 tile (fp16 2:4 512 x 1024 x 4096
// 9.8 vs 10.2 us); the 64 x 64 and 32 x 32 tiles run faster from stage 0 (int8
// 2:4 512 x 1024 x 3072 6.6 vs 6.9 us on 64 x 64; 32 x 32 with a 4-stage ring:
// fp16 2:4 512 x 1024 x 1024 5.7 vs 6.5 us, int8 2:4 512 x 4096 x 1024 9.1 vs
// 10.6 us against the rotated 3-stage form).
template <bool NTS, int NLD = 0>
using CfgBig = Cfg<4, 2, 2, 4, 3, 8, NTS, false, 0, false, NLD>;
template <bool NTS>
using CfgBigDense = Cfg<4, 2, 2, 4, 2, 8, NTS, false, 0, false, 4>;
template <bool NTS>
using CfgMid = Cfg<2, 2, 2, 4, 2, 8, NTS, false>;
template <bool NTS, bool ROT>
using CfgSmall = Cfg<2, 2, 2, 2, 3, 8, NTS, ROT>;
template <bool NTS, bool ROT, int MP>
using CfgSmallP = Cfg<2, 2, 2, 2, 3, 8, NTS, ROT, MP, true>;
template <bool NTS, bool ROT>
using CfgSmallPD2 = Cfg<2, 2, 2, 2, 3, 8, NTS, ROT, 0, true, 0, 2>;
template <bool NTS, bool ROT>
using CfgSmall2 = Cfg<2, 2, 2, 2, 2, 8, NTS, ROT>;
template <bool NTS, bool ROT>
using CfgT64 = Cfg<2, 2, 1, 1, 3, 8, NTS, ROT>;
template <bool NTS, bool ROT>
using CfgT64N = Cfg<2, 2, 1, 2, 3, 8, NTS, ROT>;
template <bool NTS, bool ROT>
using CfgT64NP = Cfg<2, 2, 1, 2, 3, 8, NTS, ROT, 4, true>;
template <bool NTS>
using CfgT32 = Cfg<1, 1, 1, 1, 4, 8, NTS, false>;

enum Shape { SHAPE_BIG, SHAPE_MID, SHAPE_SMALL, SHAPE_SMALLP, SHAPE_SMALL2, SHAPE_T64, SHAPE_T64N, SHAPE_T32 };

static long tiles(int M, int N, int bm, int bn) { return long((M + bm - 1) / bm) * long((N + bn - 1) / bn); }

// tile rows x columns of a shape
static void tile_dims(Shape sh, int &bm, int &bn) {
    bm = sh == SHAPE_BIG ? 256 : (sh == SHAPE_T64 || sh == SHAPE_T64N) ? 64 : sh == SHAPE_T32 ? 32 : 128;
    bn = (sh == SHAPE_BIG || sh == SHAPE_MID) ? 256 : sh == SHAPE_T64 ? 64 : sh == SHAPE_T32 ? 32 : 128;
}

// few output tiles: at most `limit` tiles of 128 x 128 (128 = half the CUs)
static bool few_tiles(int M, int N, long limit = 128) { return tiles(M, N, 128, 128) <= limit; }

// The smallest GEMMs (at most 512 tiles of 32 x 32, fewer than 64 K stages):
// one-wave 32 x 32 tiles.  Past 64 K stages such shapes split K on 64 x 64
// tiles instead, which is faster there (fp16 2:4 512 x 4096 x 1024: 15.6 us
// split vs 21.7 on 32 x 32).
static bool tiny(int M, int N, int stages) { return stages < 64 && tiles(M, N, 32, 32) <= 512; }

// f16 kinds: big tiles when they still give >= 3/4 of a tile per CU; 64-row
// tiles for few-tile GEMMs.
static Shape pick_f16(int M, int N, int K) {
    if (few_tiles(M, N)) {
        if (tiny(M, N, K / 64)) return SHAPE_T32;
        return tiles(M, N, 64, 64) <= 256 ? SHAPE_T64 : SHAPE_T64N;
    }
    return tiles(M, N, 256, 256) >= 192 ? SHAPE_BIG : SHAPE_SMALLP;
}

// int8 kinds.  Short K (<= 1024): the per-tile prologue and the output
// stream weigh most, so the choice follows how evenly the tiles fill the
// chip's workgroup slots (ViT-Base fc1 12608x768x3072: 1188 Mid tiles, Small2
// 45 us vs Mid 47.6; ViT-L qkv / fc1: 384 / 512 Mid tiles, Mid best; ViT-L
// proj: 128 Mid tiles, Small2 10.4 us vs Mid 14.0).  The dense kind keeps
// 2 x 96 KiB of stages for a Mid tile, i.e. one workgroup per CU, so it
// takes Small2 unless Big tiles fill the chip one to two times (ViT-L fc1).
// Long K: as the f16 kinds.
static Shape pick_i8(int M, int N, int K, bool dense) {
    // (short K: up to 192 tiles; 1024 x 1024 x 3072 2:4 9.9 -> 9.1 us, dense
    // 9.9 -> 8.1; at 256 tiles within 5 %, and with K = 4096 at 192 tiles the
    // 128-row tiles stay ahead, 20.4 vs 24.7 us)
    if (few_tiles(M, N, K <= 1024 ? 192 : 128)) return tiny(M, N, K / 128) ? SHAPE_T32 : SHAPE_T64;
    if (K <= 1024) {
        if (dense) {
            const long big = tiles(M, N, 256, 256);
            return (big >= 256 && big <= 512) ? SHAPE_BIG : SHAPE_SMALL2;
        }
        const long mid = tiles(M, N, 128, 256);
        return (mid >= 256 && mid <= 512) ? SHAPE_MID : SHAPE_SMALL2;
    }
    if (tiles(M, N, 256, 256) >= 192) return SHAPE_BIG;
    return tiles(M, N, 128, 128) <= (dense ? 576 : 256) ? SHAPE_SMALLP : SHAPE_SMALL;
}

template <int KIND, int EPI, bool NTS, bool DENSE>
static hipError_t launch_shape(Shape sh, const void *A, const void *Wv, const uint32_t *meta, const float *scale,
                               const float *bias, void *C, int M, int N, int K, hipStream_t st, int splits = 1) {
    if (sh == SHAPE_BIG) {
        if constexpr (DENSE) return launch<KIND, EPI, CfgBigDense<NTS>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
        else return launch<KIND, EPI, CfgBig<NTS, KIND == W24_F16 ? 4 : 0>>(A, Wv, meta, scale, bias, C, M, N, K, st,
                                                                          splits);
    }
    if (sh == SHAPE_MID) return launch<KIND, EPI, CfgMid<NTS>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
    constexpr bool ROT = KindTraits<KIND>::kSparse;
    if (sh == SHAPE_T64) {
        // split launches of the sparse kinds start rotated (fp16 2:4 512 x 4096
        // x 1024, 2 splits: 18.5 vs 19.4 us), unsplit ones from stage 0
        constexpr bool ROT64 = EPI == EPI_PART && KindTraits<KIND>::kSparse;
        return launch<KIND, EPI, CfgT64<NTS, ROT64>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
    }
    if (sh == SHAPE_T32) return launch<KIND, EPI, CfgT32<NTS>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
    if (sh == SHAPE_SMALLP) {
        // the int8 2:4 tile takes stages of 256 k when K allows (unsplit launches)
        if constexpr (KIND == W24_I8 && EPI != EPI_PART)
            if (K % 256 == 0)
                return launch<KIND, EPI, CfgSmallPD2<NTS, ROT>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
        constexpr int MP = !KindTraits<KIND>::kSparse ? 0 : KindTraits<KIND>::kI8 ? 2 : 4;
        return launch<KIND, EPI, CfgSmallP<NTS, ROT, MP>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
    }
    if constexpr (!KindTraits<KIND>::kI8) {  // (only the fp16 kinds pick T64N)
        if (sh == SHAPE_T64N) {
            if constexpr (KindTraits<KIND>::kSparse)
                return launch<KIND, EPI, CfgT64NP<NTS, ROT>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
            else return launch<KIND, EPI, CfgT64N<NTS, ROT>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
        }
    }
    if constexpr (KindTraits<KIND>::kI8)  // (only the int8 kinds pick Small2)
        if (sh == SHAPE_SMALL2)
            return launch<KIND, EPI, CfgSmall2<NTS, KindTraits<KIND>::kSparse>>(A, Wv, meta, scale, bias, C, M, N, K,
                                                                                st, splits);
    return launch<KIND, EPI, CfgSmall<NTS, KindTraits<KIND>::kSparse>>(A, Wv, meta, scale, bias, C, M, N, K, st, splits);
}

hipError_t launch_dense_f16(const void *A, const void *Wt, void *C, int M, int N, int K, hipStream_t st) {
    return launch_shape<DENSE_F16, EPI_F16, true, true>(pick_f16(M, N, K), A, Wt, nullptr, nullptr, nullptr, C, M, N, K,
                                                         st);
}

hipError_t launch_w24_f16(const void *A, const void *vals, const uint32_t *meta, void *C, int M, int N, int K,
                          hipStream_t st) {
    return launch_shape<W24_F16, EPI_F16, true, false>(pick_f16(M, N, K), A, vals, meta, nullptr, nullptr, C, M, N, K,
                                                        st);
}

// int8 kinds: out selects the epilogue (OUT_I32 raw accumulators; OUT_F32,
// OUT_F16 and OUT_I8 apply scale and the optional bias).  Every output kind
// keeps the int8 tile choice: with short K the main loop's operand traffic,
// not the output stream, sets most of the time (measured on the ViT-Base
// fc1 shape: fp32 / fp16 / int8 outputs 46.5 / 43.2 / 41.6 us).
template <int KIND, bool DENSE>
static hipError_t launch_i8(const void *A, const void *Wv, const uint32_t *meta, const float *scale,
                            const float *bias, void *C, int out, int M, int N, int K, hipStream_t st) {
    const Shape sh = pick_i8(M, N, K, DENSE);
    switch (out) {
        case OUT_I32:
            return launch_shape<KIND, EPI_I32, true, DENSE>(sh, A, Wv, meta, nullptr, nullptr, C, M, N, K, st);
        case OUT_F32:
            return launch_shape<KIND, EPI_F32_SCALE, true, DENSE>(sh, A, Wv, meta, scale, bias, C, M, N, K, st);
        case OUT_F16:
            return launch_shape<KIND, EPI_F16_SCALE, true, DENSE>(sh, A, Wv, meta, scale, bias, C, M, N, K, st);
        default:
            return launch_shape<KIND, EPI_I8_SCALE, true, DENSE>(sh, A, Wv, meta, scale, bias, C, M, N, K, st);
    }
}

hipError_t launch_dense_i8(const void *A, const void *Wt, const float *scale, const float *bias, void *C, int out,
                           int M, int N, int K, hipStream_t st) {
    return launch_i8<DENSE_I8, true>(A, Wt, nullptr, scale, bias, C, out, M, N, K, st);
}

hipError_t launch_w24_i8(const void *A, const void *vals, const uint32_t *meta, const float *scale, const float *bias,
                         void *C, int out, int M, int N, int K, hipStream_t st) {
    return launch_i8<W24_I8, false>(A, vals, meta, scale, bias, C, out, M, N, K, st);
}

}  // namespace ssg

namespace ssg {

// ---- split K.  The partial launches run the tile choice of the unsplit
// kinds with gridDim.y = splits and the EPI_PART epilogue (plain stores: the
// reduce launch reads the partials back right away).
// The tile of a split launch of the fp16 kinds.  Split launches read each
// weight once per tile row, cold from HBM, so where the split reaches one
// workgroup per CU with bigger tiles, those win (graph-timed, a fresh weight
// per call): fp16 2:4 512 x 4096 x 1024 16.9 us as 128 x 128 x 8 splits, 16.3
// as 64 x 128 x 4, 18.4 as 64 x 64 x 2; 512 x 8192 x 1024 21.9 / 23.2 / 30.6.
// A function of the shape and the split count alone, so an explicit split
// count gets a fixed tile too.
static Shape split_shape_f16(int M, int N, int K, int splits) {
    const Shape sh = pick_f16(M, N, K);
    if (sh != SHAPE_T64 && sh != SHAPE_T64N && sh != SHAPE_T32) return sh;
    const int S = K / 64;
    if (splits == 8 && M >= 128 && tiles(M, N, 128, 128) * 8 >= 256 && S / 8 >= 8) return SHAPE_SMALL;
    if (splits == 4 && tiles(M, N, 64, 128) * 4 >= 256 && S / 4 >= 8) return SHAPE_T64N;
    return sh;
}

hipError_t launch_gemm_partials(int kind, const void *A, const void *W, const uint32_t *meta, void *ws, int M,
                                int N, int K, int splits, hipStream_t st) {
    switch (kind) {
        case DENSE_F16:
            return launch_shape<DENSE_F16, EPI_PART, false, true>(split_shape_f16(M, N, K, splits), A, W, nullptr,
                                                                   nullptr, nullptr, ws, M, N, K, st, splits);
        case W24_F16:
            return launch_shape<W24_F16, EPI_PART, false, false>(split_shape_f16(M, N, K, splits), A, W, meta, nullptr,
                                                                  nullptr, ws, M, N, K, st, splits);
        case DENSE_I8:
            return launch_shape<DENSE_I8, EPI_PART, false, true>(pick_i8(M, N, K, true), A, W, nullptr, nullptr,
                                                                  nullptr, ws, M, N, K, st, splits);
        default:
            return launch_shape<W24_I8, EPI_PART, false, false>(pick_i8(M, N, K, false), A, W, meta, nullptr, nullptr,
                                                                 ws, M, N, K, st, splits);
    }
}

// Tile rows x columns the launchers pick for a kind and shape.
void tile_choice(int kind, int M, int N, int K, int *bm, int *bn) {
    const bool i8 = kind == DENSE_I8 || kind == W24_I8;
    const bool dense = kind == DENSE_F16 || kind == DENSE_I8;
    tile_dims(i8 ? pick_i8(M, N, K, dense) : pick_f16(M, N, K), *bm, *bn);
}

// Splitting K pays when a GEMM has few output tiles and a long K loop (one
// GPU's share of a token-sharded layer, e.g. 512 x 4096 x 1024): each tile's
// K loop is a chain of dependent stage loads, and cutting it into ranges run
// side by side shortens the chain, at the price of a second launch and the
// partials' round trip through memory (8 * M * N bytes per split).  Few-tile
// GEMMs already run on 64-row tiles (more workgroups, shorter chains per
// stage), so the split only pays from 64 K stages on.  Measured on MI355X
// with graph-timed replays on those tiles: fp16 2:4 512 x 4096 x 1024 (64
// stages, 128 tiles) 20.6 us unsplit, 15.6 with 2 splits; 128 x 4096 x 4096
// 20.2 -> 16.3; int8 2:4 512 x 8192 x 1024 21.1 -> 15.6; but with 32 stages
// (int8 512 x 4096 x 1024, fp16 256 x 2048 x 2048) 2 splits are no faster,
// and with more than 128 tiles every split loses (fp16 1024 x 4096 x 1024:
// 21.9 -> 26.5 us).  Within those bounds the splits double while tiles x
// splits stays within one workgroup per CU and every split keeps at least 8
// stages.
int suggest_splits(int kind, int M, int N, int K) {
    constexpr int kCUs = 256;
    if (M <= 0 || N <= 0 || K <= 0) return 1;
    const bool i8 = kind == DENSE_I8 || kind == W24_I8;
    const bool dense = kind == DENSE_F16 || kind == DENSE_I8;
    const Shape sh = i8 ? pick_i8(M, N, K, dense) : pick_f16(M, N, K);
    int bm, bn;
    tile_dims(sh, bm, bn);
    const long t = tiles(M, N, bm, bn);
    const int S = gemm_k_stages(kind, K);
    if (S < 64 || t > 128) return 1;
    if (!i8) {  // bigger tiles with more splits first (see split_shape_f16)
        for (int q : {8, 4})
            if (S % q == 0 && split_shape_f16(M, N, K, q) != sh) return q;
    }
    int p = 1;
    while (p < 16 && t * 2 * p <= kCUs && S % (2 * p) == 0 && S / (2 * p) >= 8) p *= 2;
    return p;
}

}  // namespace ssg
