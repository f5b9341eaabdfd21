/*
 * qmm.h -- C ABI of libqmm, the quantized-weight matmul for MI355X (gfx950).
 *
 *   out[t][r] = sum_i W[r][i] * x[t][i]
 *
 * W stays in GGUF-style super-blocks of 256 weights; x is quantized on the
 * device to int8 blocks of 32 with an f32 scale d and the f32 product
 * s = d * sum(q); each scale group of W meets one activation block and is
 * reduced as an integer dot, and the weight min folds out through the identity
 *   sum w x = d*sc*dx * sum(q*qx) - dmin*m * (dx*sum(qx)).
 *
 * Pages cited (by title, section in brackets):
 *   [GEMM] "The quantized GEMM" (mojo-dllm kernels page)
 *   [MMQ]  "llama.cpp MMQ -- quantized-weight int8 tensor-core matmul: structure,
 *          numerics, SASS census, and minfer contrast"
 *   [CH04] "04 - Reading minfer's kernels II -- from GEMV to tiled GEMM"
 *
 * Conventions (all entry points):
 *  - Pointers named W, x, q, d, s, out, S, workspace are DEVICE pointers owned by
 *    the caller; the library allocates nothing and keeps no state beyond a
 *    per-device property cache.  `stream` is a hipStream_t (NULL = default stream).
 *  - Calls are asynchronous: QMM_OK means "validated and enqueued".  Faults of
 *    the device surface at the caller's next synchronisation.
 *  - Validation happens before any device work; on an error nothing is enqueued
 *    and no output is touched.
 *  - Layouts: W row-major [od][id/256] super-blocks (row r is id/256 contiguous
 *    blocks); x token-major [nt][id] f32; q [nt][id] int8; d and s [nt][id/32] f32;
 *    out [nt][od] f32, fully overwritten.  [CH04, section 3.3]: weights arrive
 *    row-major [out][in]; [GEMM, "The shape of the problem"].
 *  - Shape rules: nt >= 1, od >= 1, id >= 256 and id % 256 == 0 (whole
 *    super-blocks); nt*id and od*(id/256) must fit in 31 bits.
 *  - Alignment: W, x, q, d, s, out and workspace must be 16-byte aligned.
 *  - Inputs must be finite (NaN/Inf behaviour is unspecified).
 *  - Only gfx950 devices are accepted (QMM_ERR_DEVICE otherwise); there is no
 *    CPU fallback and no second device path.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats.  Own ids (other tables number these types differently). */
enum {
    /* [GEMM, "The GPU path"]; [MMQ, sections 4 and 6]: 144 bytes per 256 weights:
     * f16 d | f16 dmin | 12 bytes packing eight 6-bit (scale, min) pairs | 128
     * bytes of 4-bit codes (code chunk p: byte l holds sub-block 2p low, 2p+1
     * high, position l).  w = d*sc*q - dmin*m, q in 0..15. */
    QMM_TYPE_Q4_K = 1,
    /* [GEMM, "Q6_K: the same layout and prefetch"]; [MMQ, section 4]: 210 bytes
     * per 256 weights: 128 bytes low 4-bit fields | 64 bytes high 2-bit fields |
     * 16 int8 scales (one per 16 weights) | f16 d.  w = d*sc*(q6 - 32).  The
     * element-to-bit map inside the two planes is the public GGUF arrangement
     * (two halves of 128 elements), a reading the pages leave open. */
    QMM_TYPE_Q6_K = 2,
    /* [GEMM, "The GPU path", "Weights stay in GGUF blocks"]: Q6_K with each
     * 210-byte block padded to 224 bytes at upload, so every 16-byte piece of a
     * block is aligned and the kernels read it with 16-byte loads.  Bytes 0..209
     * of a padded block are the Q6_K block; bytes 210..223 are ignored.
     * qmm_pad_q6k makes this layout from QMM_TYPE_Q6_K. */
    QMM_TYPE_Q6_K_P224 = 3,
    /* [CH03, section 3.2]: 18 bytes per 32 weights: f16 d, then 16 bytes in which
     * byte l holds element l in its low nibble and element l + 16 in its high
     * nibble; the stored nibble is round(v/d) + 8, so w = d*(nibble - 8).  [CH04,
     * section 3.4]: the offset folds out through the activation sum. */
    QMM_TYPE_Q4_0 = 4,
    /* 34 bytes per 32 weights: f16 d, then 32 int8 codes, w = d*q (the pages give
     * the block size; the layout is the public one). */
    QMM_TYPE_Q8_0 = 5,
    /* 176 bytes per 256 weights: f16 d | f16 dmin | the 12 scale bytes of Q4_K | 32
     * bytes of high bits (bit j of byte l: fifth bit of element l of sub-block j) |
     * 128 bytes of low nibbles arranged as Q4_K's.  code = nibble + 16*bit (0..31),
     * w = d*sc*code - dmin*m.  The pages name the type only; this is the public
     * layout. */
    QMM_TYPE_Q5_K = 6
    /* Every type: a row is a whole number of 256-weight groups (id % 256 == 0): one
     * super-block, or eight consecutive 32-weight blocks (144 bytes for Q4_0, 272
     * for Q8_0), so rows of the 32-weight types stay 16-byte aligned. */
};

/* Status codes. */
enum {
    QMM_OK = 0,
    QMM_ERR_ARG = -1,       /* null pointer, nt/od < 1, bad kind selector */
    QMM_ERR_TYPE = -2,      /* unknown weight type */
    QMM_ERR_SHAPE = -3,     /* id not a positive multiple of 256, or sizes too large */
    QMM_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned */
    QMM_ERR_WORKSPACE = -5, /* workspace smaller than qmm_act_bytes(nt, id) */
    QMM_ERR_DEVICE = -6,    /* current device is not gfx950, or no device */
    QMM_ERR_LAUNCH = -7,    /* a kernel launch reported an error */
    QMM_ERR_SCRATCH = -8    /* qmm_matmul_noalloc: the call needs more than its fixed scratch */
};

/* Dispatch kinds. */
enum {
    QMM_KIND_MMVQ = 1, /* nt <= switch (and 9..16 tokens on od <= 4096, see qmm_dispatch_kind):
                          weights streamed once per 8 tokens, tokens in registers */
    QMM_KIND_MMQ = 2,  /* nt > switch: tiled int8 MFMA GEMM, tile shape by cost model */
    /* MMQ with a given tile shape (qmm_matmul_q8_kind and qmm_mmq_tile only): */
    QMM_KIND_MMQ_128X64 = 3,        /* 128 rows x 64 tokens, 8 waves */
    QMM_KIND_MMQ_64X64 = 4,         /* 64 rows x 64 tokens, 4 waves */
    QMM_KIND_MMQ_64X64_SPLITK = 5,  /* 64 x 64, 8 waves in two groups splitting K */
    QMM_KIND_MMQ_WAVE32X64 = 6,     /* Q4_K only: 128 x 64, 4 waves of 32 rows x 64 tokens,
                                       weights straight into registers (the default Q4_K
                                       matrix kernel) */
    QMM_KIND_SKINNY = 7,            /* Q4_K only; up to 16 tokens per launch, more as
                                       launches on token slices of 16: 16 x 16 x 32
                                       int8 MFMA tiles of 16 weight rows x 16 tokens, the
                                       weights streamed once for all tokens ([MMQ, section
                                       12.2]: token count in registers; per-32 rescale as
                                       MMQ); qmm_matmul's kernel for Q4_K at 3..48 tokens
                                       (by shape) */
    QMM_KIND_MMQ_WAVE32X64_SPLITK = 8 /* Q4_K only (qmm_matmul_q8_kind,
                                         qmm_matmul_q8k_kind): 128 x 64, 8 waves in two
                                         groups of 4 (32 rows x 64 tokens each) taking
                                         alternate super-blocks, partial tiles added in
                                         group order */
};

/* Bytes of a [od][id] weight matrix of `type`: od*(id/256)*144 (Q4_K, Q4_0), *176
 * (Q5_K), *210 (Q6_K), *224 (Q6_K padded) or *272 (Q8_0).  0 for an unknown type or
 * a bad shape.  [GEMM, "The GPU path", "Weights stay in GGUF blocks"]: a matrix is
 * uploaded as its blocks (144 bytes per Q4_K super-block, Q6_K's 210 bytes padded to
 * 224); [CH04, section 3.4]: the weight bytes a matmul streams are rows x blocks per
 * row x bytes per block, the decode budget.  Host function, no device work. */
size_t qmm_weight_bytes(int type, int od, int id);

/* Upload-time repack: nblocks Q6_K blocks of 210 bytes (src, any alignment) to
 * the padded layout of QMM_TYPE_Q6_K_P224 (dst, 224 bytes per block, 16-byte
 * aligned; pad bytes written as zero).  src and dst must not overlap; device
 * pointers; nblocks >= 1 and nblocks * 224 < 2^40 (else QMM_ERR_SHAPE). */
int qmm_pad_q6k(const void* src, void* dst, long long nblocks, void* stream);

/* Workspace bytes qmm_matmul needs for nt tokens of id values: the q8 plane
 * (nt*id int8, rounded up to 256 B) then d and s (nt*id/32 f32 each, each rounded
 * up to 256 B).  0 for a bad shape.  [GEMM, "The GPU path", "Activations get one
 * scale per 32"]: int8 codes with one f32 scale per 32 values and scale x sum(q)
 * kept beside them; [CH04, section 3.3]: the matmul call produces that q8
 * activation plane itself before the kernel runs.  Host function, no device work. */
size_t qmm_act_bytes(int nt, int id);

/* Quantize activations to int8 blocks of 32.
 * [GEMM, "The GPU path", "Activations get one scale per 32"]; [CH04, section 2.1].
 * Per token t and block k of 32 values: amax = max|x|, d = amax/127 (IEEE f32
 * divide), q = round(x/d) with ties away from zero (IEEE divide), s = d*sum(q);
 * a block of zeros gives d = 0, q = 0, s = 0.  One wave64 handles 8 blocks with
 * 16-byte loads and cross-lane max / sum reductions.
 * x: [nt][id] f32 in; q: [nt][id] int8 out; d, s: [nt][id/32] f32 out.
 * Shape rule here: id % 32 == 0 (any id >= 32). */
int qmm_quantize_act(const float* x, int nt, int id, int8_t* q, float* d, float* s, void* stream);

/* The whole path: quantize x into `workspace`, then dispatch on nt.
 * [CH04, section 3.3]: one matmul call takes raw pointers, f32 activations, the
 * weight type and the shape, and quantizes the activations itself; invalid shapes
 * are errors, never a silent fallback.  [MMQ, section 12]: every nt has a kernel:
 * nt <= 8 (QMM_NT_SWITCH) runs MMVQ, larger nt runs MMQ (qmm_dispatch_kind).
 * workspace: device buffer of at least qmm_act_bytes(nt, id) bytes, used as
 * scratch (overwritten); ws_bytes its size.  With at least qmm_act_bytes(nt, id) +
 * qmm_streamk_ws_bytes() bytes, a call for which qmm_streamk_preferred() is 1 runs
 * the stream-K kernel (its partial tiles after the q8 plane) instead of the
 * per-tile MMQ; results then differ from the per-tile kernel's by f32 rounding
 * only, and calls sharing a workspace must not overlap in time. */
int qmm_matmul(int type, const void* W, const float* x, int nt, int od, int id, float* out,
               void* workspace, size_t ws_bytes, void* stream);

/* qmm_matmul for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * quantize, dispatch and kernels as qmm_matmul with a workspace of
 * QMM_NOALLOC_SCRATCH_BYTES, but the workspace is the library's own fixed device
 * scratch, a file-scope array of QMM_NOALLOC_SCRATCH_BYTES (32 MiB) that every device
 * the library runs on holds until the process ends.  The call allocates and frees
 * nothing.  The quantized activations take the first qmm_act_bytes(nt, id) bytes,
 * at most QMM_NOALLOC_ACT_BYTES (16 MiB; e.g. 512 tokens of 12288 values need 7.9
 * MiB), else QMM_ERR_SCRATCH before any device work; the stream-K partial tiles
 * (qmm_streamk_ws_bytes(), 16 MiB) follow them.  Nothing in the scratch needs to
 * start at zero (each call writes before it reads).  Every call on one device
 * shares that device's scratch: calls that overlap in time on one device (other
 * streams, other host threads) race and give wrong results; calls on one stream are
 * ordered and safe.  Other arguments, validation and errors as qmm_matmul. */
#define QMM_NOALLOC_SCRATCH_BYTES (32u << 20)
#define QMM_NOALLOC_ACT_BYTES (16u << 20)
int qmm_matmul_noalloc(int type, const void* W, const float* x, int nt, int od, int id, float* out,
                       void* stream);

/* The matmul on already quantized activations (reuse one quantized input for
 * several weight matrices).  q, d, s as produced by qmm_quantize_act.
 * [CH04, section 3.3]: the decode and prefill kernels read a q8 activation plane
 * that a quantize step produced or kept from an earlier call (memoized), so one
 * quantized input can serve several matmuls; [GEMM, "The GPU path", "Fused
 * elementwise kernels"]: the norm or activation feeding the matmuls ends in that
 * quantize.  Dispatch, layouts, validation and errors as qmm_matmul (no workspace:
 * the per-tile matrix kernel, never stream-K). */
int qmm_matmul_q8(int type, const void* W, const int8_t* q, const float* d, const float* s, int nt,
                  int od, int id, float* out, void* stream);

/* Same as qmm_matmul_q8 but with the kernel chosen by the caller (kind =
 * QMM_KIND_MMVQ, QMM_KIND_MMQ, or one of the QMM_KIND_MMQ_* tile shapes, the last
 * for Q4_K only, else QMM_ERR_TYPE; any nt:
 * above 8 tokens MMVQ runs one launch per slice of 8 tokens, each slice giving
 * the same bits as that slice alone).  For tests and measurement of every kernel
 * variant on one shape.  Unknown kind: QMM_ERR_ARG. */
int qmm_matmul_q8_kind(int kind, int type, const void* W, const int8_t* q, const float* d,
                       const float* s, int nt, int od, int id, float* out, void* stream);

/* Stream-K matrix kernel (Q4_K and Q6_K weights in both layouts, any nt): the
 * ntiles x (id/256) units of (128 x 64 tile, super-block) are cut into 256 equal
 * contiguous ranges, one per workgroup, so a tile count that does not fill the
 * chip still loads every CU; tiles split between workgroups are combined by a
 * second kernel that adds the partials in workgroup order (a fixed order: results
 * do not depend on timing, and differ from qmm_matmul_q8 by f32 rounding only).
 * workspace: caller's device buffer of at least qmm_streamk_ws_bytes() bytes
 * (QMM_ERR_WORKSPACE), 16-byte aligned, overwritten.  Types Q4_K, Q6_K and
 * Q6_K_P224 (others: QMM_ERR_TYPE); other rules as qmm_matmul_q8.  Calls that
 * share a workspace must not overlap in time. */
size_t qmm_streamk_ws_bytes(void);
int qmm_matmul_q8_streamk(int type, const void* W, const int8_t* q, const float* d, const float* s, int nt,
                          int od, int id, float* out, void* workspace, size_t ws_bytes, void* stream);

/* The MMQ tile shape (QMM_KIND_MMQ_128X64, _64X64 or _64X64_SPLITK) that MMQ uses
 * for this shape: the one with the fewest (rounds of workgroups over the 256 CUs)
 * x (super-blocks per wave).  Negative status for invalid shapes.  Environment
 * QMM_MMQ_TILE = 1, 2 or 3 (read once) forces one, for tuning. */
int qmm_mmq_tile(int nt, int od, int id);

/* Which kernel qmm_matmul would run for this call.  With the default switch (8):
 * QMM_KIND_SKINNY for Q4_K on 9..16 tokens of any matrix, on 3..8 tokens of a matrix
 * of at least 3072 rows, on 5..8 tokens of at least 2048 rows, on 6..8 tokens of at
 * least 1024 rows of at most 4096 columns, on 17..32 tokens of at most 12288 rows and
 * on 33..48 tokens of at most 8192 rows and 4096 columns (token slices of 16);
 * otherwise QMM_KIND_MMVQ for nt <= 8 and for 9..16
 * tokens on od <= 4096 rows (as launches on slices of 8 tokens: the MMQ tile grid
 * of such a matrix fills at most a quarter of the GPU); QMM_KIND_MMQ beyond.  With
 * another switch: QMM_KIND_MMVQ for nt <= the switch, QMM_KIND_MMQ above.  A
 * token's outputs are the same bits for every nt that runs the same kernel; the
 * kernels differ from each other by f32 rounding.  A negative status for invalid
 * arguments.  [MMQ, section 12.1]: every batch size has a dedicated
 * kernel, 1..8 tokens the quantized vector kernel and 9 and more the tiled matrix
 * kernel, with the threshold tuned per chip; [CH04, section 3.3]: the dispatch is a
 * function of nt with shape gates, and an unsupported shape is an error, not a
 * fallback.  Host function, no device work. */
int qmm_dispatch_kind(int type, int nt, int od, int id);

/* 1 if the stream-K kernel is expected to be faster than the per-tile MMQ for this
 * call, else 0; a negative status for invalid arguments.  Q4_K and Q6_K (both
 * layouts), MMQ calls only.  With T tiles of 128 x 64: never when T is a multiple
 * of 256; for T > 256 when the last round of 256 workgroups leaves at least 10 %
 * of all workgroup slots idle; for T < 256 when K has at least 32 super-blocks
 * (except T = 128: the per-tile 64 x 64 split is one full round then), or for Q6_K
 * when T <= 64.  Measured on Q4_K and Q6_K matrices of 1024..32000 rows
 * and 4096..14336 columns at 17..512 tokens.  qmm_matmul follows it when its
 * workspace is large enough. */
int qmm_streamk_preferred(int type, int nt, int od, int id);

/* The nt at or below which MMVQ (or, for Q4_K, the small-batch kernel) runs on
 * every shape (default 8; environment QMM_NT_SWITCH, clamped to 0..8, read once; a
 * value other than 8 runs MMVQ up to it and turns off the small-batch and
 * 9..16-token rules of qmm_dispatch_kind). */
int qmm_nt_switch(void);

/* For tests and tuning: force the K split of the small-batch kernel (QMM_KIND_SKINNY)
 * to ks = 1, 2, 4, 8 or 16 waves per workgroup (never more than the super-blocks of
 * a row), or 0 for the default (8, or 16 on matrices of at most 4096 rows with 32 or
 * 48 super-blocks per row).  The kernel sums over a fixed 16-way split, so its
 * results are the same bits for every ks; only its speed changes.  Process-wide, for
 * all devices and later calls; not synchronised with calls already enqueued.
 * Returns QMM_OK, or QMM_ERR_ARG for another value.  Host function, no device work. */
int qmm_set_skinny_split(int ks);

/* ---- Q8_K activations: one scale per 256 values ------------------------------
 * [GEMM, "Activations: int8 with a scale per 256"]: each activation row quantized
 * to int8 with one f32 scale per 256 values and the sum of every 16-value group of
 * codes kept as a float; [GEMM, "The zero points do not touch the inner loop"]:
 * the Q4_K min term is dmin * m times the sub-block's activation sum, read from
 * those stored sums.  Rules as qmm_quantize_act over 256 values: d = amax / 127
 * (IEEE division), q = round(x / d) half away from zero, a zero block gives
 * d = q = 0; bsum = exact sum of 16 codes (|bsum| <= 2032).  Numerics differ from
 * the per-32 path (a coarser activation scale); the results are their own. */

/* x [nt][id] f32 -> q [nt][id] int8, d [nt][id/256] f32, bsum [nt][id/16] f32.
 * id a positive multiple of 256 (QMM_ERR_SHAPE), nt >= 1 (QMM_ERR_ARG), pointers
 * device, 16-byte aligned (QMM_ERR_ALIGN), non-null (QMM_ERR_ARG). */
int qmm_quantize_act_q8k(const float* x, int nt, int id, int8_t* q, float* d, float* bsum, void* stream);

/* out [nt][od] = W x on Q8_K activations (q, d, bsum from qmm_quantize_act_q8k).
 * Per super-block b of row r and token t, Q4_K and Q5_K (codes 0..15 or 0..31):
 *   d_r * dx_tb * sum_j sc_j * sum(q * qx) - dmin_r * dx_tb * sum_j m_j * (bsum_2j + bsum_2j+1);
 * Q6_K (either layout; bsum is not read but must be a valid aligned pointer):
 *   d_r * dx_tb * sum_g sc_g * sum((q6 - 32) * qx)  over its sixteen 16-weight groups;
 * the inner sums exact integers, the f32 terms accumulated in f32.  Runs the
 * int8-MFMA matrix kernel for every nt (no vector kernel on this path).  Weight
 * types Q4_K, Q5_K, Q6_K, Q6_K_P224 (QMM_ERR_TYPE otherwise); shapes and alignment
 * as qmm_matmul_q8. */
int qmm_matmul_q8k(int type, const void* W, const int8_t* q, const float* d, const float* bsum, int nt,
                   int od, int id, float* out, void* stream);

/* qmm_matmul_q8k with the tile shape chosen by the caller: kind = QMM_KIND_MMQ
 * (the rule of qmm_q8k_tile), QMM_KIND_MMQ_128X64, QMM_KIND_MMQ_64X64 or
 * QMM_KIND_MMQ_64X64_SPLITK (two groups of waves take alternate super-blocks and
 * add their partial tiles in group order at the end), and for Q4_K only
 * (QMM_ERR_TYPE otherwise) QMM_KIND_MMQ_WAVE32X64 or QMM_KIND_MMQ_WAVE32X64_SPLITK:
 * 4 waves of 32 rows x 64 tokens per 128 x 64 tile, each sub-block scale split as
 * sc = 8a + b with a, b <= 7 and carried inside the int8 weight operand (a q and
 * b q are at most 105), so two int32 accumulators chained over the super-block
 * give sum_j sc_j * sum(q * qx) = 8 Ca + Cb exactly ([GEMM, "Activations: int8
 * with a scale per 256"]: one activation scale per super-block makes that sum a
 * single integer).  Same results bit for bit as QMM_KIND_MMQ_128X64 and
 * QMM_KIND_MMQ_64X64_SPLITK respectively.  qmm_matmul_q8k runs the unsplit one for
 * Q4_K wherever there are more than 256 tiles of 128 x 64.
 * For tests and measurement.  Other kinds: QMM_ERR_ARG; other rules as
 * qmm_matmul_q8k. */
int qmm_matmul_q8k_kind(int kind, int type, const void* W, const int8_t* q, const float* d, const float* bsum,
                        int nt, int od, int id, float* out, void* stream);

/* The tile shape (QMM_KIND_MMQ_128X64, _64X64 or _64X64_SPLITK) qmm_matmul_q8k uses
 * for this shape: the one with the fewest (rounds of workgroups over the 256 CUs)
 * x (super-blocks per wave), ties to the larger tile, as qmm_mmq_tile.  Negative
 * status for invalid shapes. */
int qmm_q8k_tile(int nt, int od, int id);

/* Diagnostic: the integer stage of qmm_matmul_q8k alone.  S [nt][od][id/256][2]
 * int32: S[..][0] = sum_j sc_j * sum(q * qx), S[..][1] = sum_j m_j * (bsum_2j +
 * bsum_2j+1) (Q4_K, Q5_K); S[..][0] = sum_g sc_g * sum((q6 - 32) * qx), S[..][1] =
 * 0 (Q6_K), computed by the code of the kernel qmm_matmul_q8k takes for the shape
 * (for Q4_K with more than 256 tiles of 128 x 64: the wave kernel's 8 Ca + Cb).
 * Arguments as qmm_matmul_q8k. */
int qmm_q8k_superblock_sums(int type, const void* W, const int8_t* q, const float* d, const float* bsum,
                            int nt, int od, int id, int32_t* S, void* stream);

/* ---- Producer-side steps fused with the quantizer ---------------------------
 * [GEMM, "The GPU path", "Fused elementwise kernels"]: each RMS norm and the FFN
 * activation ends in the quantizer; fusing them removes the HBM write and re-read
 * of the f32 rows.  The fused calls give bit for bit what the unfused chain gives
 * (the same float expressions in the same order, the same quantizer code):
 *   qmm_add_rmsnorm_quantize  = qmm_residual_add, qmm_rmsnorm, qmm_quantize_act
 *   qmm_rmsnorm_quantize      = qmm_rmsnorm, qmm_quantize_act
 *   qmm_silu_mul_quantize     = qmm_silu_mul, qmm_quantize_act
 * One quantized activation serves every projection that reads it (q, k, v from
 * one norm; gate and up from another) through qmm_matmul_q8.
 *
 * Arithmetic (the pages fix only that fused equals unfused):
 *   RMS norm, f32: lane partials p_t (t = 0..255) accumulate fma(x_i, x_i, p_t) in
 *   increasing i over the i with (i / 4) mod 256 == t; they are combined by halving,
 *   p_t += p_{t+s} for s = 128, 64, ..., 1, giving ss; r = 1 / sqrtf(ss / id + eps);
 *   y_i = (x_i * r) * w_i.
 *   silu(g) * u: (g / (1 + exp(-g))) * u evaluated in f64, rounded once to f32.
 *
 * Common rules: rows are [nt][id] f32, id % 32 == 0 (id >= 32); q [nt][id] int8,
 * d and s [nt][id/32] f32 as from qmm_quantize_act; w [id] f32; every pointer a
 * device pointer owned by the caller, 16-byte aligned (QMM_ERR_ALIGN), non-null
 * (QMM_ERR_ARG); nt < 1: QMM_ERR_ARG; id not a positive multiple of 32, or
 * nt * id >= 2^31: QMM_ERR_SHAPE; eps negative, infinite or NaN: QMM_ERR_ARG.
 * eps = 0 with an all-zero row is outside the domain (0 * infinity).  Inputs
 * must be finite and the results finite.  Asynchronous on `stream`. */

/* h <- h + o (the residual stream, updated in place), then the RMS norm of the
 * new h times w, quantized into q, d, s.  o may equal h. */
int qmm_add_rmsnorm_quantize(float* h, const float* o, const float* w, float eps, int nt, int id,
                             int8_t* q, float* d, float* s, void* stream);

/* The RMS norm of x times w, quantized into q, d, s (a layer whose input needs
 * no residual add). */
int qmm_rmsnorm_quantize(const float* x, const float* w, float eps, int nt, int id, int8_t* q,
                         float* d, float* s, void* stream);

/* silu(g) * u, elementwise over [nt][id], quantized into q, d, s. */
int qmm_silu_mul_quantize(const float* g, const float* u, int nt, int id, int8_t* q, float* d,
                          float* s, void* stream);

/* The same three steps ending in the Q8_K quantizer (qmm_quantize_act_q8k's rules;
 * id a multiple of 256, else QMM_ERR_SHAPE): q [nt][id] int8, d [nt][id/256],
 * bsum [nt][id/16] f32, bit for bit the unfused step followed by
 * qmm_quantize_act_q8k.  For the Q8_K matrix path (qmm_matmul_q8k). */
int qmm_add_rmsnorm_quantize_q8k(float* h, const float* o, const float* w, float eps, int nt, int id, int8_t* q,
                                 float* d, float* bsum, void* stream);
int qmm_rmsnorm_quantize_q8k(const float* x, const float* w, float eps, int nt, int id, int8_t* q, float* d,
                             float* bsum, void* stream);
int qmm_silu_mul_quantize_q8k(const float* g, const float* u, int nt, int id, int8_t* q, float* d, float* bsum,
                              void* stream);

/* Unfused steps (f32 out), the chain the fused calls are equal to. */
/* h <- h + o over [nt][id] (id % 32 == 0 as above). */
int qmm_residual_add(float* h, const float* o, int nt, int id, void* stream);
/* y = RMS norm of x times w; y may equal x. */
int qmm_rmsnorm(const float* x, const float* w, float eps, int nt, int id, float* y, void* stream);
/* y = silu(g) * u. */
int qmm_silu_mul(const float* g, const float* u, int nt, int id, float* y, void* stream);

/* Diagnostic: the integer stage of a kernel alone.  [GEMM, "The GPU path"]: each
 * scale group (32 weights for Q4_K, Q5_K, Q4_0 and Q8_0, 16 for Q6_K) is reduced as
 * an integer dot with its activation codes.  Writes S[t][r][b][g] = sum over group g
 * of 256-weight group b of row r of (code * qx) -- codes 0..15 (0..31) uncentred for
 * Q4_K (Q5_K),
 * (q6 - 32) for Q6_K, (nibble - 8) for Q4_0, the int8 for Q8_0 -- as int32,
 * computed by the unpack and dot code of the kernel `kind` (QMM_KIND_MMVQ: v_dot4
 * path, nt <= 8; QMM_KIND_MMQ: int8 MFMA path).
 * S: [nt][od][id/256][8 or 16] int32, 16-byte aligned. */
int qmm_group_dots(int kind, int type, const void* W, const int8_t* q, int nt, int od, int id,
                   int32_t* S, void* stream);

/* Diagnostic: one MFMA tile with the operand and result lane mapping the MMQ
 * kernels rely on, written out as C[.][token][row], for a test that pins the
 * layouts.  kind 1: int8 32x32x32; A [32 rows][32 K] int8, B [32 tokens][32 K] int8,
 * C [32 tokens][32 rows] int32 = B . A^T.  kind 2: f32 pair of 32 x 32 outer
 * products; A [2][32 rows] f32, B [2][32 tokens] f32, C [2][32 tokens][32 rows] f32.
 * kind 3: f32 32x32x2; A [2 K][32 rows], B [2 K][32 tokens] f32, C [32 tokens][32
 * rows] f32 = sum over K.  All buffers device, 16-byte aligned. */
int qmm_mfma_tile_check(int kind, const void* A, const void* B, void* C, void* stream);

/* Short text for a status code (static storage). */
const char* qmm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
