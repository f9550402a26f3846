/*
 * woq.h - C ABI of libwoq: weight-only quantised linear layers for LLM decode
 * on AMD MI355X (gfx950).
 *
 * Two weight formats are supported.
 *
 *  INT8  - symmetric per-tensor quantisation: scale = max|W| / 127 and
 *          code = round(W / scale), reconstructed as code * scale ("Open Origin -
 *          ELG Stream Layer" README, Technical Architecture: "INT8 Quantization
 *          & Direct Mapping" and "FP16 On-The-Fly GPU Reconstruction").
 *  INT4O - outlier-aware INT4 ("On-The-Fly Weight Synthesizer (OTF-LLM Engine)",
 *          Architecture & Key Innovations, the architecture diagram and item 3):
 *          a global input-channel permutation puts the top 1% of channels by
 *          |W| x |X_profile| at the end and keeps them as FP16; the other 99%
 *          are INT4 codes in [-7, 7] with zero-point 0, packed two per byte,
 *          with one fp16 scale per output row per 128 background channels; the
 *          output is X_out W_out^T + X_bg deq(W_bg)^T.
 *
 * Conventions for every entry point.
 *  - Matrices are row-major.  A weight is [N, K] (N output features, K input
 *    features); activations are x [b, K] and outputs y [b, N].
 *  - fp16 values cross the ABI as uint16_t bit patterns.
 *  - Rounding is IEEE round-to-nearest-even everywhere (W / scale is an fp32
 *    division; a code is the nearest integer, ties to even, then clamped to
 *    +-127 or +-7).
 *  - Every function returns an int status (WOQ_OK or a negative WOQ_E* code).
 *    Arguments are checked before any work starts; on an error nothing is
 *    written.  No C++ exception crosses the ABI.
 *  - Host functions are synchronous, run on the calling thread plus a pool of
 *    worker threads (WOQ_NUM_THREADS, default min(16, hardware threads)) and
 *    give bit-identical results for any thread count.
 *  - Device functions are asynchronous on the caller's stream (a hipStream_t
 *    passed as void*; NULL is the default stream).  Pointers are device memory
 *    owned by the caller and must stay valid until the stream reaches the
 *    work.  Vector-loaded pointers must be 16-byte aligned (WOQ_EALIGN
 *    otherwise).  A launch failure returns WOQ_EHIP (see woq_last_hip_error);
 *    a fault inside a kernel surfaces at the caller's next synchronisation.
 *  - Buffer extents: a device entry point sees only pointers, so it cannot
 *    check the size of a buffer.  Every activation or output buffer must hold
 *    at least the b rows of its leading dimension that the call names (b * ld
 *    fp16 values, the last row at least its used width); a shorter buffer is
 *    read or written out of bounds by the kernel.
 *  - The library allocates no memory visible to the caller, except inside the
 *    opaque runtime objects, which own their buffers until destroyed.
 */
#ifndef WOQ_H
#define WOQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */

#define WOQ_OK            0
#define WOQ_EINVAL       (-1)  /* bad argument: null pointer, negative or inconsistent size */
#define WOQ_EALIGN       (-2)  /* pointer or leading dimension not aligned as required */
#define WOQ_ENOMEM       (-3)  /* host or device allocation failed (runtime objects only) */
#define WOQ_EHIP         (-4)  /* a HIP call failed; woq_last_hip_error() gives its code */
#define WOQ_EUNSUPPORTED (-5)  /* valid request that the library does not implement */
#define WOQ_ERANGE       (-6)  /* value not representable: non-finite weight, fp16 scale overflow */
#define WOQ_EIO          (-8)  /* a file could not be opened, read or written */
#define WOQ_EFORMAT      (-9)  /* not a pool file, or a damaged one (magic, version, sizes or checksum) */

#define WOQ_ABI_VERSION 1

/* Static English text for a status code (never NULL). */
const char* woq_strerror(int status);
/* hipError_t of the last failing HIP call on this thread (0 if none). */
int woq_last_hip_error(void);
/* WOQ_ABI_VERSION of the built library. */
int woq_abi_version(void);

/* ---------------------------------------------------------------- geometry */

/*
 * Sizes of the outlier split of one input space of width K.
 *   canonical: K_bg = K - n_out background channels in G = ceil(K_bg/128)
 *              groups, zero-padded to K_pad = 128 * G.
 *   device   : G4 = G rounded up to a multiple of 4, n_out8 = n_out rounded
 *              up to a multiple of 8; a permuted activation row (woq_permute_x)
 *              holds xp_len = 128 * G4 + n_out8 fp16 values: the background
 *              channels, zeros up to 128 * G4, the outlier channels, zeros.
 */
typedef struct {
    int64_t K, n_out, K_bg, G, K_pad;
    int64_t G4, n_out8, xp_len;
} woq_int4o_geom;

/* Fill *g for an input space of width K >= 1 with 0 <= n_out <= K outlier
 * channels.  n_out < 0 selects the default ceil(K/100) (the pages' 1%). */
int woq_int4o_geometry(int64_t K, int64_t n_out, woq_int4o_geom* g);

/* ------------------------------------------------------------ host: INT8 */

/*
 * Quantise W (float32 [N, K]) with one fp32 scale for the whole tensor:
 * *scale = fp32(max|W| / 127), q = clamp(rne(fp32(W / *scale)), -127, 127).
 * An all-zero tensor (or one whose scale underflows to 0) gives *scale = 0 and
 * q = 0.  WOQ_ERANGE if W holds a NaN or an infinity.  q is int8 [N, K].
 * ("Open Origin - ELG Stream Layer", Technical Architecture: the scale and
 * int8 equations.)
 */
int woq_quantize_int8(const float* W, int64_t N, int64_t K, int8_t* q, float* scale);

/* ----------------------------------------------------------- host: INT4O */

/*
 * colsum[j] += sum_n |W[n, j]| in float64, for every input channel j of one
 * linear (W float32 [N, K]).  Call once for every linear of every layer that
 * reads the input space, then woq_outlier_select.  The sum over n runs in
 * row order for each j, whatever the thread count.
 */
int woq_colabs_accumulate(const float* W, int64_t N, int64_t K, double* colsum);

/*
 * Global static permutation of one input space ("On-The-Fly Weight
 * Synthesizer (OTF-LLM Engine)", item 3): score_j = mean_t |xprof[t, j]| *
 * colsum[j] in float64 (xprof fp16 [T, K], T >= 1); the n_out channels with the
 * largest score (ties to the lower index) are the outliers.  perm (int32 [K])
 * receives the background channels in ascending order followed by the outlier
 * channels in ascending order.  n_out < 0 selects ceil(K/100).  WOQ_ERANGE if
 * a profile value or a score is not finite.
 */
int woq_outlier_select(const double* colsum, const uint16_t* xprof, int64_t T, int64_t K,
                       int64_t n_out, int32_t* perm);

/*
 * The whole selection for one input space in one call (item 3's single table
 * for the model): colsum = the sum over the n_lin linears that read the space
 * (every layer) of their column sums sum_n |W_l[n, j]|, each linear's sum
 * formed from zero in row order and the linears added in the order given,
 * all in float64; then woq_outlier_select.  Ws[l] is float32 [Ns[l], K].
 * Bit-identical to woq_outlier_perm_sums over woq_colabs_accumulate sums of
 * the same linears, in the same order, each into a zeroed buffer.
 */
int woq_outlier_perm(const float* const* Ws, const int64_t* Ns, int32_t n_lin, int64_t K, const uint16_t* xprof,
                     int64_t T, int64_t n_out, int32_t* perm);

/*
 * woq_outlier_perm for callers that cannot hold every weight of the space at
 * once (a model generated or loaded layer by layer): parts[i] (float64 [K])
 * are per-linear column sums, each from woq_colabs_accumulate into a zeroed
 * buffer; they are added in the order given (parts[0] first), then the
 * selection runs as woq_outlier_select.  n_parts >= 1.
 */
int woq_outlier_perm_sums(const double* const* parts, int32_t n_parts, int64_t K, const uint16_t* xprof,
                          int64_t T, int64_t n_out, int32_t* perm);

/*
 * Outlier-aware INT4 encoding of W (float32 [N, K], original channel order)
 * under perm (int32 [K], as from woq_outlier_select) with n_out outlier
 * channels (n_out < 0: ceil(K/100)).  Writes the canonical arrays:
 *   packed uint8 [N, K_pad/2]  - byte j of a row holds the code of permuted
 *                                background channel 2j in its low nibble and
 *                                2j+1 in its high nibble, two's complement,
 *                                zero codes in the padding;
 *   scales fp16  [N, G]        - scale of group g = fp16(fp32(max|W_g| / 7))
 *                                over the group's real channels;
 *   w_out  fp16  [N, n_out]    - fp16(W[:, perm[K_bg + i]]).
 * Codes are clamp(rne(fp32(W / fp32(scale))), -7, 7), or 0 where the scale is 0.
 * WOQ_ERANGE for a non-finite weight or a scale that overflows fp16;
 * WOQ_EINVAL if perm is not a permutation of 0..K-1.
 */
int woq_quantize_int4o(const float* W, int64_t N, int64_t K, const int32_t* perm, int64_t n_out,
                       uint8_t* packed, uint16_t* scales, uint16_t* w_out);

/* Unpack canonical packed codes (uint8 [N, K_pad/2]) to int8 [N, K_pad]. */
int woq_unpack_int4(const uint8_t* packed, int64_t N, int64_t K_pad, int8_t* q);

/* ---------------------------------------------------- host: device layouts */

/*
 * INT8 device layout: N4 = N rounded up to 4 rows, Kd = K rounded up to 64
 * columns; row-major [N4, Kd] bytes holding code + 128 (offset binary), with
 * code 0 in the padding.  woq_int8_dev_bytes gives the size.
 */
int64_t woq_int8_dev_bytes(int64_t N, int64_t K);
int woq_layout_int8(const int8_t* q, int64_t N, int64_t K, uint8_t* dev);
int woq_layout_int8_inverse(const uint8_t* dev, int64_t N, int64_t K, int8_t* q);

/*
 * INT4O device layout, in tiles of 16 rows (N16 = N rounded up to 16; padding
 * rows hold code 0, scale 0 and zero outlier weights):
 *   codes  : for each tile, group g (0 .. G4-1) and 32-channel chunk c (0..3)
 *            of the group, 256 bytes: 16 bytes per row of the tile, row-minor.
 *            The 16 bytes of (row, g, c) hold the codes of background channels
 *            128g + 32c + 16P + t (P = 0, 1; t = 0..15) as offset-binary
 *            nibbles (code + 8), dword e (0, 1) of half P holding, at nibble
 *            positions 0,4,2,6 the channels t = 4e+0..4e+3 and at positions
 *            1,5,3,7 the channels t = 8+4e+0..8+4e+3.  A (tile, group) block is
 *            1 KB; a row's codes are 64 * G4 bytes.
 *   scales : [N16/16][G4][16] fp16 - the 16 rows of a tile side by side per group.
 *   w_out  : [N16/16][n_out8/8][16] chunks of 8 fp16 (the outlier weights of
 *            channels 8i .. 8i+7 of each row, row-minor within a tile), zero-padded.
 * Byte sizes from woq_int4o_dev_sizes.  The inverse reproduces the canonical
 * arrays bit for bit.
 */
int woq_int4o_dev_sizes(int64_t N, const woq_int4o_geom* g, int64_t* codes_bytes,
                        int64_t* scales_bytes, int64_t* wout_bytes);
int woq_layout_int4o(const uint8_t* packed, const uint16_t* scales, const uint16_t* w_out, int64_t N,
                     const woq_int4o_geom* g, uint8_t* dev_codes, uint16_t* dev_scales,
                     uint16_t* dev_wout);
int woq_layout_int4o_inverse(const uint8_t* dev_codes, const uint16_t* dev_scales,
                             const uint16_t* dev_wout, int64_t N, const woq_int4o_geom* g,
                             uint8_t* packed, uint16_t* scales, uint16_t* w_out);

/* ------------------------------------------------- device: encoders (prep) */

/*
 * The INT8 encoding of woq_quantize_int8 computed on the device, written
 * straight into the INT8 device layout (woq_layout_int8), bit for bit what the
 * host functions give.  W: fp32 [N, K] row-major in device memory (4-byte
 * aligned); dev: woq_int8_dev_bytes(N, K) bytes (16-byte aligned); *scale
 * (device fp32) receives the scale - it doubles as the running maximum while
 * the call runs; *status (device int32) receives 0, or WOQ_ERANGE if W holds a
 * NaN or an infinity (then *scale is NaN and every code 0).  Asynchronous on
 * stream: four launches (maximum, codes, scale, status clear).  For weights
 * that already sit in device memory or arrive layer by layer: the host keeps
 * no copy (the bounded-memory prep of "On-The-Fly Weight Synthesizer
 * (OTF-LLM Engine)", item 2, done by the GPU).
 */
int woq_quantize_int8_dev(const float* W, int64_t N, int64_t K, uint8_t* dev, float* scale, int32_t* status,
                          void* stream);

/*
 * The outlier-aware INT4 encoding of woq_quantize_int4o under perm (device
 * int32 [g->K]) computed on the device, written straight into the INT4O
 * device layout (woq_layout_int4o; sizes from woq_int4o_dev_sizes, each array
 * 16-byte aligned; an array of size 0 may be null), bit for bit what
 * the host functions give.  W: fp32 [N, g->K] row-major in device memory.
 * *status (device int32) receives 0; WOQ_ERANGE for a non-finite weight or a
 * group scale that overflows fp16; WOQ_EINVAL for a permutation entry outside
 * [0, K) (that entry reads as 0; a repeated entry is not detected - perm must
 * come from woq_outlier_select).  Asynchronous on stream.
 */
int woq_quantize_int4o_dev(const float* W, int64_t N, const int32_t* perm, const woq_int4o_geom* g,
                           uint8_t* dev_codes, uint16_t* dev_scales, uint16_t* dev_wout, int32_t* status,
                           void* stream);

/* ----------------------------------------------------------- device ops */

#define WOQ_MAX_SEGMENTS 8

/*
 * An INT8 weight resident in device memory (woq_layout_int8 of N rows).  Rows
 * [seg_end[i-1], seg_end[i]) use seg_scale[i] (seg_end[-1] = 0,
 * seg_end[nseg-1] = N): one segment for a single linear, several for linears
 * that read the same input and are stacked along N into one launch.
 */
typedef struct {
    const void* codes;
    int64_t N, K;
    int32_t nseg;
    int64_t seg_end[WOQ_MAX_SEGMENTS];
    float seg_scale[WOQ_MAX_SEGMENTS];
} woq_int8_w;

/* An INT4O weight resident in device memory (woq_layout_int4o of N rows). */
typedef struct {
    const void* codes;
    const void* scales;
    const void* w_out;
    int64_t N;
    woq_int4o_geom geom;
} woq_int4o_w;

/*
 * Permute and split activations for an INT4O input space (the architecture
 * diagram's "Global Static Permutation" and its outlier / background split):
 * xp[r, k] = x[r, perm[k]] for k < K_bg, 0 for K_bg <= k < 128*G4,
 * xp[r, 128*G4 + i] = x[r, perm[K_bg + i]] for i < n_out, 0 up to n_out8.
 * x fp16 [b, ldx] (ldx >= K), perm int32 [K] in device memory, xp fp16
 * [b, g->xp_len] (16-byte aligned); x and xp must hold all b rows.  b = 0 is
 * a no-op.
 */
int woq_permute_x(const uint16_t* x, int64_t ldx, const int32_t* perm, int64_t b,
                  const woq_int4o_geom* g, uint16_t* xp, void* stream);

/*
 * y[r, n] = fp16(scale(n) * sum_k code[n, k] * x[r, k]) for r < b, n < N, with
 * fp32 accumulation, reading the INT8 codes once from HBM and converting them
 * in registers (the reconstruction step of "Open Origin - ELG Stream Layer",
 * fused into the product).  x fp16 [b, ldx], 16-byte aligned, ldx a multiple
 * of 8 and >= K; y fp16 [b, ldy], ldy >= N; x and y must hold all b rows.
 * 1 <= b <= 8 (b = 0 is a no-op).
 * The vector-ALU kernel runs, except for N >= 16384 at b >= 4 and N >= 8192
 * at b >= 7, where a matrix-core kernel runs (the faster one on MI355X).
 */
int woq_qgemv_int8(const woq_int8_w* w, const uint16_t* x, int64_t ldx, int64_t b,
                   uint16_t* y, int64_t ldy, void* stream);

/*
 * INT8 vocabulary lookup ("On-The-Fly Weight Synthesizer (OTF-LLM Engine)",
 * Architecture & Key Innovations, item 4: vocabulary tables held as INT8; each
 * looked-up row restored as in "Open Origin - ELG Stream Layer", "FP16
 * On-The-Fly GPU Reconstruction"):
 *   y[r, k] = fp16(fp32(code[ids[r], k] * scale(ids[r])))   for r < b, k < K,
 * the product rounded to fp32 and then to fp16, both to nearest even.  w is the
 * table (N = vocabulary rows, K = hidden width) in the INT8 device layout;
 * ids int32 [b] in device memory (4-byte aligned); y fp16 [b, ldy], 16-byte
 * aligned, ldy a multiple of 8 and >= K.  A row whose id lies outside [0, N)
 * is written as zeros (ids are device data, so they cannot be checked before
 * the launch).  b <= 65535; b = 0 is a no-op.
 */
int woq_embed_int8(const woq_int8_w* w, const int32_t* ids, int64_t b, uint16_t* y, int64_t ldy,
                   void* stream);

/*
 * y[r, n] = fp16(sum_i w_out[n, i] xp[r, 128*G4 + i]
 *               + sum_g scale[n, g] sum_{k in g} code[n, k] xp[r, k])
 * with fp32 accumulation ("On-The-Fly Weight Synthesizer (OTF-LLM Engine)",
 * architecture diagram: the outlier GEMM and the fused background GEMM added
 * into one FP16 output).  xp from woq_permute_x (fp16 [b, xp_len]); y fp16
 * [b, ldy], ldy >= N; xp and y must hold all b rows.  The vector-ALU kernel
 * runs for b <= 2, and for b <= 4 when N <= 6128 (fewer than 384 tiles of 16 rows), if b * (2 * xp_len +
 * 16 * G4) bytes (the staged activations and a correction per 32-channel
 * chunk) fit in 62 KB of LDS; otherwise the matrix-core kernel
 * (woq_qgemm_int4o) runs - on MI355X the faster of the two in each case.
 * 1 <= b <= 64 (b = 0 is a no-op).
 */
int woq_qgemv_int4o(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y,
                    int64_t ldy, void* stream);

/*
 * Positions of the input channels in the permuted, padded activation row of
 * woq_permute_x: pos[j] = k such that xp[r, k] = x[r, j] (host function).
 * pos holds round_up(K, 8) entries; entries K.. are 0xFFFF.  WOQ_EINVAL if
 * perm is not a permutation of [0, K); WOQ_EUNSUPPORTED if xp_len > 65535.
 */
int woq_perm_positions(const int32_t* perm, const woq_int4o_geom* g, uint16_t* pos);

/*
 * woq_permute_x and woq_qgemv_int4o in one launch - the same result bit for
 * bit wherever woq_qgemv_int4o runs its vector kernel (b <= 2, or b <= 4 when
 * N <= 6128), the same values up to summation order where it runs the
 * matrix-core kernel: x is read in its natural channel order (fp16 [b, ldx],
 * all b rows, 16-byte aligned, ldx a multiple of 8 and >= K; y as for
 * woq_qgemv_int4o) and scattered through pos (device
 * copy of woq_perm_positions, 16-byte aligned) into the permuted, split row,
 * held in on-chip memory while the weights stream; this is the vector-ALU
 * kernel of woq_qgemv_int4o at any 1 <= b <= 4.  WOQ_EUNSUPPORTED unless
 * woq_qgemv_int4o_x_supported(g, b) (1 <= b <= 4, xp_len <= 65535 and
 * b * (2 * xp_len + 16 * G4) bytes fit 62 KB); callers then use the
 * two-call form.
 */
int woq_qgemv_int4o_x(const woq_int4o_w* w, const uint16_t* x, int64_t ldx, const uint16_t* pos,
                      int64_t b, uint16_t* y, int64_t ldy, void* stream);
int woq_qgemv_int4o_x_supported(const woq_int4o_geom* g, int64_t b);

/*
 * woq_permute_x and woq_qgemm_int4o in one launch, on the matrix cores: the
 * same result bit for bit (the same plans, groups, matrix-core steps and
 * reductions).  x is read in its natural channel order (fp16 [b, ldx], all b
 * rows, 16-byte aligned, ldx a multiple of 8 and >= K; y as for
 * woq_qgemm_int4o); each workgroup scatters it through pos (device copy of
 * woq_perm_positions, 16-byte aligned) into the whole permuted, split row of
 * its 8 staged batch columns, held in on-chip memory (16 bytes per 8
 * channels of the padded row, about 130 KB at K = 8192) while the weights
 * stream, so the permutation needs no launch of its own (the OTF-LLM page's
 * global static permutation, "Architecture & Key Innovations", applied
 * where the product reads its input).  WOQ_EUNSUPPORTED unless
 * woq_qgemm_int4o_x_supported(g, N, b): 1 <= b <= 8, rows of 64 groups or
 * more, xp_len <= 65535, the staged row fits the device's LDS per workgroup
 * and the product's workgroups (one per compute unit) fit the device in one
 * round; callers then use the two-call form.  Asynchronous on stream.
 */
int woq_qgemm_int4o_x(const woq_int4o_w* w, const uint16_t* x, int64_t ldx, const uint16_t* pos,
                      int64_t b, uint16_t* y, int64_t ldy, void* stream);
int woq_qgemm_int4o_x_supported(const woq_int4o_geom* g, int64_t N, int64_t b);

/* The matrix-core (MFMA) kernel of woq_qgemv_int4o for any 1 <= b <= 64
 * (xp and y as there: all b rows). */
int woq_qgemm_int4o(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y,
                    int64_t ldy, void* stream);

/*
 * woq_qgemm_int4o with the groups of every row split into `splits` K ranges
 * (1..16) that run as separate workgroups covering more rows each, so that
 * each staged activation chunk serves more weights; each range's fp32 partial
 * sums go to workspace (device memory, 16-byte aligned, at least
 * woq_qgemm_int4o_splitk_workspace(N, b, splits) bytes, owned by the caller;
 * its contents on return are unspecified), and a second launch adds the
 * ranges in a fixed order into y.  The same result as woq_qgemm_int4o up to
 * summation order, deterministic for a given split count.  Calls that share
 * a workspace must not overlap.
 */
int woq_qgemm_int4o_splitk(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y, int64_t ldy,
                           int32_t splits, float* workspace, int64_t workspace_bytes, void* stream);
int64_t woq_qgemm_int4o_splitk_workspace(int64_t N, int64_t b, int32_t splits);

/*
 * woq_qgemm_int4o_splitk for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The partial sums go to a fixed workspace of
 * WOQ_SPLITK_NOALLOC_BYTES that the library keeps in device memory of its own
 * (one per device, held from the library's first use of that device until the
 * process ends); the call allocates nothing.  splits * b * N * 4 bytes must fit
 * in it: WOQ_EUNSUPPORTED otherwise (8 MiB holds 8 splits of the 70B-shaped
 * down product, N = 8192, up to b = 32).  Every call on one device shares that
 * workspace, which keeps the last call's partial sums: calls that overlap on
 * one device (different streams without synchronisation, or threads) race
 * and give wrong results.  Same results as woq_qgemm_int4o_splitk bit for bit.
 */
#define WOQ_SPLITK_NOALLOC_BYTES (8 << 20)
int woq_qgemm_int4o_splitk_noalloc(const woq_int4o_w* w, const uint16_t* xp, int64_t b, uint16_t* y, int64_t ldy,
                                   int32_t splits, void* stream);

/* --------------------------------------------------------- layer stack */

#define WOQ_FMT_INT8  1
#define WOQ_FMT_INT4O 2

/*
 * One step of a decode stack: a (possibly N-stacked) linear that reads input
 * slot in_slot and writes output slot out_slot.  fmt selects w8 or w4; an
 * INT4O step also names the device permutation of its input space (int32
 * [geom.K]).  Slots index the pointer arrays given to woq_stack_run.
 */
typedef struct {
    int32_t fmt;
    int32_t in_slot, out_slot;
    woq_int8_w w8;
    woq_int4o_w w4;
    const int32_t* perm;
} woq_stack_step;

typedef struct woq_stack woq_stack;

/*
 * Create a runner for n_steps steps executed in order on one stream ("Open
 * Origin - ELG Stream Layer", Key Features 2: each layer's cycle, and the
 * OTF-LLM runner that drives the model through the fused kernels).  The step
 * array is copied; the weights it points to stay owned by the caller.  The
 * runner owns an activation workspace for batches up to max_b (allocated on
 * the current device here) and, for each distinct INT4O permutation, a device
 * channel-position table (woq_perm_positions), built here from the
 * permutation's device copy, which must therefore hold its values already.
 * WOQ_EINVAL if a permutation is not one; WOQ_ENOMEM if an allocation fails.
 */
int woq_stack_create(const woq_stack_step* steps, int32_t n_steps, int64_t max_b, woq_stack** out);

/*
 * Run every step once, in order, on `stream`: an INT4O step is one
 * woq_qgemv_int4o_x launch wherever its vector kernel serves the batch and
 * that form applies (woq_qgemv_int4o_x_supported, K a multiple of 8, the
 * input 16-byte aligned), one woq_qgemm_int4o_x launch wherever the
 * matrix-core kernel serves it without a K split and that form applies
 * (woq_qgemm_int4o_x_supported, K a multiple of 8, the input 16-byte
 * aligned), otherwise woq_permute_x followed by the matrix-core product
 * (woq_qgemm_int4o; on rows of 128 groups or more at 9 <= b <= 32 its
 * split-K form, woq_qgemm_int4o_splitk with 8 ranges and a runner-owned
 * workspace, two launches); an INT8 step is one woq_qgemv_int8 launch.  The
 * one-launch and two-launch forms give the same bits.
 * inputs[slot] are fp16 [b, K of the step]
 * activations (rows contiguous), outputs[slot] fp16 [b, N of the step]; the
 * two pointer arrays must have an entry for every slot a step names, and each
 * buffer must hold those b rows (the runner sees pointers only).
 * 1 <= b <= max_b.  Asynchronous; the caller synchronises.  Every run of
 * one runner writes the same workspace (permuted activations, split-K
 * partial sums), so runs of one runner must not overlap: issue them on one
 * stream, or synchronise between streams.
 */
int woq_stack_run(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                  void* stream);

/*
 * Kernel launches of one woq_stack_run pass at batch b (a folded INT4O step
 * or an INT8 step is one launch, a permute-then-product INT4O step two, three
 * with the split-K reduction), assuming 16-byte aligned inputs.
 */
int woq_stack_launches(const woq_stack* st, int64_t b, int32_t* launches);

/*
 * woq_stack_run repeated `iters` times with a pair of HIP events around every
 * step and around every pass.  A step's events take the dispatch timestamps
 * of its own launches: the start of its first launch (the permutation, where
 * one precedes the product) and the end of its last (the split-K reduction,
 * where one follows).  On return (the stream is synchronised) step_ms[i]
 * (n_steps floats) holds the mean duration of step i and *pass_ms the mean
 * duration of one pass.  Dispatch-boundary spans of consecutive launches can
 * overlap by part of the dispatch time, so the step durations may add up to
 * a little more than the pass.  For measurement only; iters >= 1.
 */
int woq_stack_time(woq_stack* st, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                   void* stream, int32_t iters, float* step_ms, float* pass_ms);

/* Release the runner and its workspace (after the stream has finished). */
int woq_stack_destroy(woq_stack* st);

/* ------------------------------------------------------- streamed pager */

/*
 * One product of a streamed INT8 layer: its device-layout codes start
 * code_offset bytes into the layer's block; w gives N, K and the segment
 * scales (w.codes is ignored).
 */
typedef struct {
    int64_t code_offset;
    woq_int8_w w;
} woq_pager_step;

typedef struct woq_pager woq_pager;

/*
 * Tier plan under a device-memory budget (NTransformer summary, "3-Tier
 * Adaptive Caching Architecture": tier A layers stay resident in device
 * memory, tier B layers live in pinned host memory and are streamed in by
 * host-to-device DMA; host function).  Layers are taken in order: layers
 * 0 .. n_A-1 are resident, the rest streamed, with n_A the largest count for
 * which the resident bytes plus, when any layer streams, two slots of the
 * largest streamed block fit budget_bytes.  Resident layers come first so that
 * the first copies overlap their products.  resident[l] (int32 [n_layers])
 * receives 1 or 0; *device_bytes (may be null) the bytes the plan places in
 * device memory.  WOQ_ENOMEM if not even two slots fit; WOQ_EINVAL if a layer
 * has no bytes.
 */
int woq_plan_tiers(const int64_t* layer_bytes, int32_t n_layers, int64_t budget_bytes, int32_t* resident,
                   int64_t* device_bytes);

/*
 * Tiered decode pass over n_layers layers of steps_per_layer products each
 * (steps in layer order; each step reads inputs[in_slot] and writes
 * outputs[out_slot] of woq_pager_run, as woq_stack_run does).  Layer l is
 * resident when layer_bytes[l] == 0: its steps hold device pointers.  Otherwise
 * it is streamed: its block is layer_bytes[l] bytes at pinned_pool +
 * layer_off[l] (page-locked memory from hipHostMalloc or an equivalent pinned
 * allocation, owned by the caller, valid while the pager exists), and the
 * weight pointers of its steps (w8.codes; w4.codes, w4.scales, w4.w_out) hold
 * byte offsets into that block instead of addresses, each 16-byte aligned with
 * its array inside the block (WOQ_EINVAL otherwise).  INT8 and INT4O steps may
 * be mixed as in woq_stack_create, whose limits apply (max_b <= 8 with INT8
 * steps, <= 64 otherwise).  The pager allocates two device slots of the
 * largest streamed block, its events and the stack runner's workspace.
 */
int woq_tiered_create(const void* pinned_pool, const int64_t* layer_off, const int64_t* layer_bytes,
                      int32_t n_layers, const woq_stack_step* steps, int32_t steps_per_layer, int64_t max_b,
                      woq_pager** out);

/*
 * Streamed decode over INT8 layers that all live in pinned host memory ("Open
 * Origin - ELG Stream Layer", Key Features 1-3: a block-allocated INT8 pool in
 * pinned RAM, asynchronous layer paging, double-buffered prefetch of layer N+1
 * on a secondary stream while layer N computes): woq_tiered_create with every
 * layer streamed, step s of layer l an INT8 product whose codes start
 * code_offset bytes into the layer's block, reading inputs[l * steps_per_layer
 * + s] and writing outputs[l * steps_per_layer + s].  1 <= max_b <= 8.
 */
int woq_pager_create(const void* pinned_pool, const int64_t* layer_off, const int64_t* layer_bytes,
                     int32_t n_layers, const woq_pager_step* steps, int32_t steps_per_layer, int64_t max_b,
                     woq_pager** out);

/*
 * One pass: on copy_stream, the j-th streamed layer's block is copied into
 * slot j mod 2 once the products of streamed layer j-2 have finished with
 * that slot (the first two copies start at once, behind any work already
 * queued on compute_stream); on compute_stream, the layers run in order, a
 * streamed layer's products once its copy has landed.  The two streams must
 * be distinct when any layer streams; both are left with work queued
 * (synchronise compute_stream to wait for the outputs).  Passes of one pager
 * must not overlap.
 */
int woq_pager_run(woq_pager* p, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                  void* compute_stream, void* copy_stream);

/* Number of streamed (tier B) layers of a pager. */
int woq_pager_streamed_layers(const woq_pager* p, int32_t* n);

/*
 * One woq_pager_run pass with HIP events on the copy stream around every
 * block copy (for measurement).  For the j-th streamed layer, wait_ms[j] is
 * when the copy stream reached it (before waiting for its slot), copy_ms[j]
 * when the copy started (the slot was free) and end_ms[j] when the copy had
 * landed, all in milliseconds from the pass's start on the compute stream;
 * *pass_ms is the pass's duration on the compute stream.  The arrays hold
 * woq_pager_streamed_layers entries (null when there are none).  Synchronises
 * both streams.
 */
int woq_pager_time(woq_pager* p, const uint16_t* const* inputs, uint16_t* const* outputs, int64_t b,
                   void* compute_stream, void* copy_stream, float* wait_ms, float* copy_ms, float* end_ms,
                   float* pass_ms);

/* Release the slots, events and workspace (after both streams have finished). */
int woq_pager_destroy(woq_pager* p);

/* ------------------------------------------------------ persisted pool */

/*
 * A pool file holds the encoded layer blocks of a stack (device layouts, as
 * streamed by the tiered pass) and opaque caller metadata, so that a later
 * process loads them instead of encoding the weights again - the persisted
 * INT8 pool of "Open Origin - ELG Stream Layer" (its first boot quantises and
 * saves, later boots load), for either format.  Host functions; synchronous.
 * Each block sits at a 4096-byte aligned offset with a 64-bit checksum (FNV-1a
 * over 8-byte words of each 1 MiB chunk, then over the chunk hashes); the
 * table and the metadata carry a checksum of their own.  Reads and writes use
 * up to 16 threads.
 */

/* Write the file at path (replaced if it exists).  blocks[i] (host memory,
 * pinned or not) of block_bytes[i] bytes.  WOQ_EIO on a file error. */
int woq_pool_save(const char* path, const void* meta, int64_t meta_bytes, const void* const* blocks,
                  const int64_t* block_bytes, int32_t n_blocks);

/* Read the table: *n_blocks and *meta_bytes; the first max_blocks block sizes
 * into block_bytes and the first meta_cap metadata bytes into meta (either may
 * be null).  WOQ_EFORMAT for a file that is not an intact pool header. */
int woq_pool_info(const char* path, int32_t* n_blocks, int64_t* meta_bytes, int64_t* block_bytes,
                  int32_t max_blocks, void* meta, int64_t meta_cap);

/* Read block i into dst (host memory of dst_bytes >= the block's size; pinned
 * memory serves a later DMA directly) and verify its checksum: WOQ_EFORMAT on
 * a mismatch or a truncated file (dst then holds what was read). */
int woq_pool_read_block(const char* path, int32_t i, void* dst, int64_t dst_bytes);

/* ------------------------------------------------------------ measurement */

/*
 * Read `bytes` bytes (a multiple of 16, 16-byte aligned device memory) with
 * one 16-byte non-temporal load per lane and chunk, the way the products
 * stream their weights, and discard them: the achievable streaming-read rate
 * against which the products' bandwidth is reported.  Asynchronous on
 * `stream`; the caller times it.  bytes = 0 is a no-op.
 */
int woq_stream_read(const void* buf, int64_t bytes, void* stream);

/*
 * Launch `iters` empty kernels of `blocks` workgroups of `threads` threads on
 * `stream` twice over and report, in microseconds: *span_us, the mean time
 * between each launch's own dispatch-boundary events (the events the stack
 * runner's timing pass records around each step; consecutive spans overlap by
 * part of the dispatch), and *interval_us, the mean time per launch when they
 * run back to back with one pair of events around all of them (what each
 * dependent launch adds to a pass before its own work).  Synchronises the
 * stream.  1 <= blocks, 1 <= threads <= 1024, 1 <= iters <= 100000.
 */
int woq_dispatch_floor(int32_t blocks, int32_t threads, int32_t iters, void* stream, float* span_us,
                       float* interval_us);

#ifdef __cplusplus
}
#endif

#endif /* WOQ_H */
