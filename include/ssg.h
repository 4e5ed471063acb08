/*
 * ssg.h -- C ABI of libssg: structured-sparse weight GEMM for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes C = A x W for a pruned linear layer (A: M x K
 * activations, W: K x N weight, C: M x N) with W sparse in one of two
 * patterns:
 *
 *   2:4    at most two nonzeros in every group of four consecutive K entries
 *          of an output column.  GPUSQ-ViT ("Boost Vision Transformer with
 *          GPU-Friendly Sparsity and Quantization", abstract) prunes to this
 *          pattern for fp16 and then quantises for the integer 2:4 path.
 *   TW     tile-wise: W is cut into tiles of G consecutive output columns
 *          spanning all of K; each tile keeps its own whole rows and columns
 *          ("Accelerating Sparse DNN Models without Hardware-Support via
 *          Tile-Wise Sparsity", tile-wise pattern slide) and runs as a
 *          condensed dense tile whose A rows are read through offset_k and
 *          whose C columns are written through offset_n (run-time slide).
 *
 * The pages split the method into offline preprocessing and a run-time GEMM
 * fed by the preprocessed arrays; the ABI mirrors that split:
 *
 *   - pack functions: host, synchronous, CPU only.  Every pointer is
 *     caller-owned host memory.
 *   - GEMM / transpose functions: asynchronous on `stream` (a hipStream_t
 *     passed as void*; NULL = the legacy default stream).  Every pointer is
 *     caller-owned device memory of the current HIP device, contiguous and
 *     16-byte aligned.  Nothing is allocated.  The call returns after the
 *     launch is enqueued; results are visible after the stream synchronises.
 *
 * Conventions for every function:
 *   - the return value is a status code (SSG_OK = 0);
 *   - on failure nothing has been written to any output or enqueued, except
 *     SSG_EHIP from a failed launch;
 *   - arguments are validated on the host before any HIP call; a failure
 *     returns SSG_EINVAL (or the code named below) and sets a message that
 *     ssg_last_error() returns on the same thread;
 *   - packed arrays handed to a GEMM are trusted: offsets or positions out of
 *     range are undefined behaviour (they are not re-validated on device);
 *   - all functions are re-entrant; the only state is a per-device cache of
 *     the architecture check and the thread-local error message.
 *
 * Shapes are int64_t element counts.  fp16 data travel as uint16_t bit
 * patterns on the host side and as untyped device pointers.
 */
#ifndef SSG_H
#define SSG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SSG_OK = 0,
    SSG_EINVAL = 1, /* bad shape, alignment, pointer or parameter            */
    SSG_ENOT24 = 2, /* a 4-group holds more than two nonzeros                */
    SSG_ENOSPC = 3, /* caller capacity smaller than tw_pack_query's result   */
    SSG_ENODEV = 4, /* no HIP device visible                                 */
    SSG_EARCH = 5,  /* current device is not gfx950                          */
    SSG_EHIP = 6    /* a HIP runtime call or kernel launch failed            */
};

/* Message describing the last failing call on this thread ("" if none).
 * The pointer stays valid until the next failing call on the same thread. */
const char *ssg_last_error(void);

/* Library version string, e.g. "ssg 0.1.0 gfx950". */
const char *ssg_version(void);

/* Writes the current device's architecture name (e.g. "gfx950:sramecc+:xnack-")
 * into buf (NUL-terminated, truncated to len).  SSG_ENODEV without a device. */
int ssg_device_arch(char *buf, int64_t len);

/* ------------------------------------------------------------------------
 * 2:4 pack stage (GPUSQ-ViT abstract: 2:4 fine-grained structured pruning,
 * FP16 and integer).  The pages fix no storage format; this one is:
 *
 *   W     [K][N] row-major (N contiguous), the densified pruned weight W_p.
 *   vals  [N][K/2]: for column n and group g (k = 4g .. 4g+3) the two kept
 *         values in slots 2g, 2g+1, in ascending k.  Zeros are stored as +0.
 *   meta  [N][ceil(K/32)] uint32: slot j of column n holds its position in
 *         the group (0..3) at bits 2*(j%16) of word j/16.
 *
 * Kept positions: the group's nonzero positions (-0.0 counts as zero),
 * topped up with its lowest-index zero positions to exactly two, ascending.
 * Requires K % 4 == 0, K > 0, N > 0.  A group with more than two nonzeros
 * returns SSG_ENOT24 naming the first offending (group, column).
 * ------------------------------------------------------------------------ */
int w24_pack_f16(const uint16_t *W, int64_t K, int64_t N, uint16_t *vals, uint32_t *meta);
int w24_pack_i8(const int8_t *W, int64_t K, int64_t N, int8_t *vals, uint32_t *meta);

/* Inverse: W[4g + pos][n] = vals[n][slot]; every other entry +0.
 * Positions are checked (each group's two positions must be distinct and
 * ascending) and a violation returns SSG_EINVAL. */
int w24_unpack_f16(const uint16_t *vals, const uint32_t *meta, int64_t K, int64_t N, uint16_t *W);
int w24_unpack_i8(const int8_t *vals, const uint32_t *meta, int64_t K, int64_t N, int8_t *W);

/* ------------------------------------------------------------------------
 * Tile-wise pack stage ("Accelerating Sparse DNN Models without
 * Hardware-Support via Tile-Wise Sparsity": offline re-organisation into
 * condensed tiles, run-time GEMM through offset_k / offset_n).
 *
 * Tile t covers output columns [t*G, min(N, t*G+G)), T = ceil(N/G).
 *   offset_n  kept columns of tile t, tile-local, ascending (columns with a
 *             nonzero in the tile);
 *   offset_k  kept rows of tile t, global k, ascending (rows with a nonzero
 *             among the tile's columns);
 *   vals      tile t's block V_t[j][kk] = W[offset_k[kk]][t*G + offset_n[j]],
 *             stored [N_t][ld_t] with ld_t = K_t rounded up so that a row is
 *             a multiple of 16 bytes (8 fp16 or 16 int8 elements; zero
 *             padded), tiles back to back;
 *   v_ptr, k_ptr, n_ptr  [T+1] prefix sums (elements of vals, of offset_k,
 *             of offset_n);
 *   tile_order [T] tiles by K_t*N_t descending, ties to the lower t
 *             (longest-processing-time order for the grouped launch).
 * tw_pack_query (tw_pack_query_i8) fills the sizes; tw_pack_f16
 * (tw_pack_i8) returns SSG_ENOSPC when a capacity in *cap is smaller than
 * needed.  The int8 forms are the same format with int8 values (the
 * quantised deployment of the integer path).  Requires G > 0, K > 0, N > 0,
 * K < 2^31, and sum of tile sizes < 2^31.
 * tw_unpack_f16 (tw_unpack_i8) writes the dense W [K][N] (pruned entries +0)
 * after checking the arrays against each other: prefix sums starting at 0
 * and non-decreasing, each tile's vals span equal to N_t * ld_t, offsets in
 * range (offset_k < K, offset_n < the tile's width), no null array of
 * nonzero length; a violation returns SSG_EINVAL with nothing written.
 * ------------------------------------------------------------------------ */
typedef struct {
    int64_t T;          /* number of tiles                 */
    int64_t sum_kt;     /* length of offset_k              */
    int64_t sum_nt;     /* length of offset_n              */
    int64_t vals_elems; /* length of vals (padded rows)    */
} tw_sizes;

int tw_pack_query(const uint16_t *W, int64_t K, int64_t N, int32_t G, tw_sizes *out);
int tw_pack_f16(const uint16_t *W, int64_t K, int64_t N, int32_t G, const tw_sizes *cap,
                uint16_t *vals, int32_t *offset_k, int32_t *offset_n,
                int32_t *v_ptr, int32_t *k_ptr, int32_t *n_ptr, int32_t *tile_order);
int tw_unpack_f16(const uint16_t *vals, const int32_t *offset_k, const int32_t *offset_n,
                  const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                  int64_t K, int64_t N, int32_t G, uint16_t *W);
int tw_pack_query_i8(const int8_t *W, int64_t K, int64_t N, int32_t G, tw_sizes *out);
int tw_pack_i8(const int8_t *W, int64_t K, int64_t N, int32_t G, const tw_sizes *cap,
               int8_t *vals, int32_t *offset_k, int32_t *offset_n,
               int32_t *v_ptr, int32_t *k_ptr, int32_t *n_ptr, int32_t *tile_order);
int tw_unpack_i8(const int8_t *vals, const int32_t *offset_k, const int32_t *offset_n,
                 const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                 int64_t K, int64_t N, int32_t G, int8_t *W);

/* ------------------------------------------------------------------------
 * Device GEMMs (gfx950 only: SSG_EARCH elsewhere, SSG_ENODEV without a GPU).
 * A is [M][K] row-major (K contiguous); C is [M][N] row-major.
 * M >= 1 is arbitrary; M == 0 is a no-op returning SSG_OK.
 * ------------------------------------------------------------------------ */

/* Dense baseline, fp16 in, fp32 accumulate, fp16 out (round to nearest even).
 * Wt is the weight stored [N][K] (K contiguous).  K % 64 == 0, N % 64 == 0.
 * The pages' dense baseline is a vendor GEMM ("Accelerating Sparse DNN
 * Models ..." pattern-comparison table); this is the same-shape MFMA one. */
int dense_gemm_f16(const void *A, const void *Wt, void *C,
                   int64_t M, int64_t N, int64_t K, void *stream);

/* Dense baseline, int8 in, int32 accumulate.  scale == NULL: C is int32 [M][N].
 * Otherwise C is fp32 [M][N] with C = float(acc) * scale[n] (each step
 * rounded to nearest even, no fused multiply-add).  K % 128 == 0, N % 64 == 0. */
int dense_gemm_i8(const int8_t *A, const int8_t *Wt, const float *scale, void *C,
                  int64_t M, int64_t N, int64_t K, void *stream);

/* 2:4 GEMM, fp16 in, fp32 accumulate, fp16 out (nearest even), from the
 * packed vals / meta of w24_pack_f16.  Runs on the gfx950 sparse matrix
 * cores, which pick the matching activations by the 2-bit positions.
 * K % 64 == 0, N % 64 == 0. */
int w24_gemm_f16(const void *A, const void *vals, const uint32_t *meta, void *C,
                 int64_t M, int64_t N, int64_t K, void *stream);

/* 2:4 GEMM, int8 in, exact int32 accumulate; epilogue as dense_gemm_i8
 * (scale == NULL -> int32 C, else fp32 C = float(acc) * scale[n]).
 * K % 128 == 0, N % 64 == 0. */
int w24_gemm_i8(const int8_t *A, const int8_t *vals, const uint32_t *meta, const float *scale,
                void *C, int64_t M, int64_t N, int64_t K, void *stream);

/* Output kinds of the int8 GEMMs' selectable epilogue. */
enum {
    SSG_OUT_I32 = 0, /* raw int32 accumulators; scale and bias must be NULL      */
    SSG_OUT_F32 = 1, /* fp32 y                                                    */
    SSG_OUT_F16 = 2, /* fp16 y, rounded to nearest even (overflow gives +-inf)   */
    SSG_OUT_I8 = 3   /* int8: y rounded to nearest even, saturated to [-128,127] */
};

/* int8 GEMMs (dense baseline and 2:4) with a lower-traffic epilogue.  The
 * integer path of GPUSQ-ViT ("Boost Vision Transformer with GPU-Friendly
 * Sparsity and Quantization", abstract) deploys the 2:4 model with integer
 * kernels; an output of 2 or 1 bytes per element, which the next quantised
 * layer consumes, moves a half or a quarter of the fp32 output's bytes.
 *
 *   y[m][n] = float(acc[m][n]) * scale[n]  (+ bias[n] when bias != NULL)
 *
 * computed in fp32, each step rounded to nearest even (the int32 -> fp32
 * conversion, the product, the sum; no fused multiply-add), then stored as
 * out_type says.  scale: fp32 [N], required except for SSG_OUT_I32; bias:
 * fp32 [N] or NULL (must be NULL for SSG_OUT_I32); both 16-byte aligned.
 * C: [M][N] elements of the out_type.  Shape rules as dense_gemm_i8 /
 * w24_gemm_i8; an unknown out_type is SSG_EINVAL.  dense_gemm_i8 and
 * w24_gemm_i8 are these calls with bias = NULL and out_type SSG_OUT_F32
 * (scale given) or SSG_OUT_I32 (scale NULL). */
int dense_gemm_i8_out(const int8_t *A, const int8_t *Wt, const float *scale, const float *bias,
                      void *C, int32_t out_type, int64_t M, int64_t N, int64_t K, void *stream);
int w24_gemm_i8_out(const int8_t *A, const int8_t *vals, const uint32_t *meta, const float *scale,
                    const float *bias, void *C, int32_t out_type, int64_t M, int64_t N, int64_t K,
                    void *stream);

/* ------------------------------------------------------------------------
 * Split K, for GEMMs whose output tiles leave most of the chip idle (one
 * GPU's share of a token-sharded layer, e.g. M = 512 rows).  The K loop of
 * every output tile is cut into `splits` equal ranges run by separate
 * workgroups; each writes its raw accumulators (fp32 for the fp16 kinds,
 * int32 for the int8 kinds) to its [M][N] slice of the workspace, and a
 * second kernel on the same stream sums the slices in split order and
 * applies the kind's epilogue.  int8 results equal the unsplit calls' bit
 * for bit (the int32 sum is the accumulator itself); fp16 results differ
 * from theirs only in the fp32 summation order, within the same bound.  The
 * pages' kernels split no reduction; this is a scheduling choice for
 * MI355X's 256 CUs.
 *
 * kind: SSG_KIND_*.  splits: 1..64 and a divisor of the K stages (K/64 for
 * the fp16 kinds, K/128 for the int8 kinds); splits == 1 runs the unsplit
 * kernel and ignores ws.  ws: device memory of at least
 * ssg_splitk_workspace_bytes(M, N, splits) bytes (ws_bytes says how many),
 * 16-byte aligned, owned by the caller; its contents are ignored and
 * overwritten, and nothing else may use it until this call's work on
 * `stream` has completed.  Every other argument and rule as in the unsplit
 * call of the same kind.  Nothing is allocated; errors as the unsplit calls
 * (SSG_EINVAL for bad splits or a short or misaligned workspace).
 * ------------------------------------------------------------------------ */
enum { SSG_KIND_DENSE_F16 = 0, SSG_KIND_W24_F16 = 1, SSG_KIND_DENSE_I8 = 2, SSG_KIND_W24_I8 = 3 };

/* Workspace bytes of a split call: splits * M * N * 4 (0 for splits <= 1 or
 * negative sizes). */
int64_t ssg_splitk_workspace_bytes(int64_t M, int64_t N, int32_t splits);

/* The split count the library would take for a kind and shape (measured on
 * MI355X): 1 (do not split) when K has fewer than 64 stages (64 K elements
 * per stage for the fp16 kinds, 128 for int8) or the output tiles of the
 * library's tile choice number more than 128.  Otherwise, for the fp16
 * kinds, 8 when 128 x 128 tiles x 8 splits reach 256 workgroups (M >= 128,
 * >= 8 stages per split), else 4 when 64 x 128 tiles x 4 do; failing both,
 * and for the int8 kinds, the largest power of two <= 16 with tiles x splits
 * <= 256 (one workgroup per CU) and at least 8 K stages per split.  A split
 * launch of the fp16 kinds uses those bigger tiles when called with that
 * split count (8 or 4) and the same conditions hold, otherwise the unsplit
 * call's tile.  Host-only; an invalid kind or shape gives 1. */
int32_t ssg_splitk_suggest(int32_t kind, int64_t M, int64_t N, int64_t K);

/* The output tile the GEMM calls of a kind use for a shape (measured choice,
 * see the tile notes of the GEMM kernels): rows * 1024 + columns, rows and
 * columns each one of 32, 64, 128, 256.  256 x 256 once such tiles give about
 * a tile per CU; when the output has at most 128 tiles of 128 x 128 (192 for
 * the int8 kinds with K <= 1024): 32 x 32 if those number at most 512 and K
 * has fewer than 64 stages (64 K elements per stage for fp16, 128 for int8),
 * else 64 x 64 (64 x 128 for the fp16 kinds when 64 x 64 tiles would
 * outnumber the 256 CUs);
 * otherwise 128 x 128 or 128 x 256.  This is the tile of the unsplit launch
 * (the plain GEMM calls, and the *_splitk calls with splits == 1); a split
 * launch of the fp16 kinds may take 128 x 128 (8 splits) or 64 x 128 (4
 * splits) tiles instead, as ssg_splitk_suggest describes.  Host-only; 0 for
 * an invalid kind or shape. */
int32_t ssg_tile_choice(int32_t kind, int64_t M, int64_t N, int64_t K);

int dense_gemm_f16_splitk(const void *A, const void *Wt, void *C, int64_t M, int64_t N, int64_t K,
                          int32_t splits, void *ws, int64_t ws_bytes, void *stream);
int w24_gemm_f16_splitk(const void *A, const void *vals, const uint32_t *meta, void *C,
                        int64_t M, int64_t N, int64_t K, int32_t splits, void *ws, int64_t ws_bytes,
                        void *stream);
int dense_gemm_i8_splitk(const int8_t *A, const int8_t *Wt, const float *scale, const float *bias,
                         void *C, int32_t out_type, int64_t M, int64_t N, int64_t K, int32_t splits,
                         void *ws, int64_t ws_bytes, void *stream);
int w24_gemm_i8_splitk(const int8_t *A, const int8_t *vals, const uint32_t *meta, const float *scale,
                       const float *bias, void *C, int32_t out_type, int64_t M, int64_t N, int64_t K,
                       int32_t splits, void *ws, int64_t ws_bytes, void *stream);

/* Allocation-free variant of w24_gemm_f16_splitk, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The partial
 * accumulators go to a static device array of SSG_STATIC_SCRATCH_BYTES
 * (32 MiB) that the library holds on every GPU it runs on until the process
 * ends; the call itself allocates nothing.  Arguments, results and errors as
 * w24_gemm_f16_splitk, without ws / ws_bytes; splits * M * N * 4 above the
 * scratch size is SSG_EINVAL.  Every call on one GPU shares that GPU's
 * scratch: calls that may overlap in time on one GPU (different streams,
 * or threads) race and must be ordered by the caller; calls on one stream
 * are ordered by the stream.  The scratch needs no clearing: each split
 * writes its whole slice before the reduction reads it. */
#define SSG_STATIC_SCRATCH_BYTES (32 << 20)
int w24_gemm_f16_splitk_static(const void *A, const void *vals, const uint32_t *meta, void *C,
                               int64_t M, int64_t N, int64_t K, int32_t splits, void *stream);

/* Tile-wise GEMM, fp16 in, fp32 accumulate, fp16 out.  At is A stored
 * K-major ([K][M], M contiguous) so that the rows picked by offset_k are
 * contiguous reads (the tile-wise slides transpose A to avoid uncoalesced
 * access).  The packed arrays are tw_pack_f16's, in device memory, with
 * T = ceil(N/G).  Every column of C is written: kept columns get the tile
 * product, pruned columns +0.  Requires G % 16 == 0, G <= 256, N % G == 0,
 * M >= 0, K >= 1; At, vals and C 16-byte aligned.  Any M is accepted: when M
 * is not a multiple of 8 the rows of At are not 16-byte aligned and the
 * kernel gathers them through registers (slower than the direct-to-LDS
 * loads of the aligned case); tiles wider than 128 columns run a wider
 * configuration (two workgroups per CU instead of three).  A caller that
 * knows every tile keeps at most 64 columns gets the faster narrow-tile
 * kernels through tw_gemm_f16_ex with SSG_TW_NARROW (same result, bit for
 * bit). */
int tw_gemm_f16(const void *At, const void *vals, const int32_t *offset_k,
                const int32_t *offset_n, const int32_t *v_ptr, const int32_t *k_ptr,
                const int32_t *n_ptr, const int32_t *tile_order, int32_t T, int32_t G,
                void *C, int64_t M, int64_t N, int64_t K, void *stream);

/* Flags of tw_gemm_f16_ex. */
enum {
    SSG_TW_OUT_T = 1,      /* write C transposed: Ct [N][M], M contiguous            */
    SSG_TW_A_ROWMAJOR = 2, /* the A argument is row-major A [M][K], not At [K][M]    */
    SSG_TW_NARROW = 4      /* the caller promises every tile keeps <= 64 columns     */
};

/* Tile-wise GEMM over a range of tiles, optionally with transposed output.
 * Runs the tiles tile_order[t_first .. t_first + t_count) (0 <= t_first,
 * t_count >= 1, t_first + t_count <= T) and writes only their G-column
 * windows of C; every other argument is as in tw_gemm_f16.
 *   - flags & SSG_TW_OUT_T: C is Ct [N][M] (row n = output channel, tokens
 *     contiguous), i.e. the K-major input At of a following tile-wise layer.
 *     The tile-wise slides fuse A's transpose into the producing kernel (the
 *     BERT layer); here the producing tile-wise GEMM writes its output in
 *     that layout, so chained tile-wise layers need no separate transpose.
 *   - a tile range lets the caller run condensed tiles as separate launches
 *     (for example one per stream, as the slides' multi-stream scheduling
 *     does); tw_gemm_f16 is one launch over all tiles in LPT order.
 *   - flags & SSG_TW_A_ROWMAJOR: the first argument is A [M][K] row-major
 *     (16-byte aligned), read without a transpose: the slides' "without
 *     transpose" case, whose gathered activations are scattered 2-byte
 *     accesses (it exists to measure that cost; K-major At is the fast path).
 *   - flags & SSG_TW_NARROW: the caller states that every tile it runs keeps
 *     at most 64 columns (n_ptr[t+1] - n_ptr[t] <= 64; the host packer knows
 *     this, the library cannot see it without reading device memory).  The
 *     kernel then sizes its stage buffers and registers for 64 columns, so
 *     more work items share a CU (and, in launches of at most two items per
 *     CU with K >= 2048, K-major At and M % 8 == 0, it takes 64 picked rows
 *     per stage).
 *     Honoured for G <= 128 and ignored for wider tiles.  A tile that keeps
 *     more than 64 columns despite the flag gets its whole output window
 *     written as quiet NaN (0x7e00), never a partial or stale result.
 *     Otherwise the results are bit-identical to the call without the flag:
 *     the same matrix instructions run over the same k order.
 * Unknown flag bits or an empty or out-of-range tile range give SSG_EINVAL. */
int tw_gemm_f16_ex(const void *At, const void *vals, const int32_t *offset_k,
                   const int32_t *offset_n, const int32_t *v_ptr, const int32_t *k_ptr,
                   const int32_t *n_ptr, const int32_t *tile_order, int32_t T, int32_t G,
                   int32_t t_first, int32_t t_count, int32_t flags, void *C,
                   int64_t M, int64_t N, int64_t K, void *stream);

/* Tile-wise GEMM, int8 in, exact int32 accumulate: the tile-wise format
 * (tw_pack_i8's arrays) on the integer path of GPUSQ-ViT ("Boost Vision
 * Transformer with GPU-Friendly Sparsity and Quantization", abstract).  At
 * is int8 A stored K-major ([K][M], M contiguous).  The epilogue is that of
 * the int8 GEMMs: out_type SSG_OUT_I32 writes the raw accumulators (scale
 * and bias NULL), otherwise y = float(acc) * scale[n] (+ bias[n]) stored as
 * fp32, fp16 or saturated int8 (scale, bias: fp32 [N], 16-byte aligned).
 * Every column of C is written: pruned columns get the epilogue of a zero
 * accumulator (0 * scale[n] + bias[n]).  Requires G % 16 == 0, G <= 256,
 * N % G == 0, M >= 0, K >= 1 (when M is not a multiple of 16 the rows of At
 * are gathered through registers, as for tw_gemm_f16). */
int tw_gemm_i8(const int8_t *At, const int8_t *vals, const int32_t *offset_k,
               const int32_t *offset_n, const int32_t *v_ptr, const int32_t *k_ptr,
               const int32_t *n_ptr, const int32_t *tile_order, int32_t T, int32_t G,
               const float *scale, const float *bias, void *C, int32_t out_type,
               int64_t M, int64_t N, int64_t K, void *stream);

/* Explicit transpose At[k][m] = A[m][k] (fp16), the "explicit transpose"
 * variant of the tile-wise slides.  M % 8 == 0, K % 8 == 0. */
int ssg_transpose_f16(const void *A, void *At, int64_t M, int64_t K, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSG_H */
