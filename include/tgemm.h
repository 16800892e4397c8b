/*
 * tgemm.h -- C ABI of libtgemm: tiled fp16 GEMM with fp32 accumulation and an
 * optional fused ReLU epilogue, C = ReLU(A @ B), on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one of "Writing High-Performance Kernels in TileLang, from
 * GEMM to MLA" (atlascloud.ai), section "Let's write a GEMM": A is M x K, B is K x N,
 * C is M x N, all IEEE binary16; the accumulator is float32 and is cleared before the
 * K loop; ReLU is max(x, 0) applied to the float32 sum; the result is written back as
 * binary16 (round to nearest even). Without ReLU it is the plain GEMM of
 * "TileLang-MUSA operator development" (7yue.com), section 3.
 *
 * Conventions for every entry point below:
 *   - Row-major storage: element (i, j) of X lives at X[i * ldX + j] (in elements).
 *   - A, B, C are DEVICE pointers on the current HIP device, owned by the caller.
 *     C must not overlap A or B. The library allocates nothing per call and keeps
 *     no state beyond an immutable config table and a per-device architecture check.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream). Calls only
 *     enqueue work and return; kernel completion and any device fault surface at the
 *     caller's next synchronisation, as usual in HIP.
 *   - ReLU maps x to x if x > 0, else +0 (so -0 and NaN become +0).
 *   - Nothing is printed, nothing aborts, no exception crosses the ABI; errors are
 *     returned as the negative codes below, detected before any work is enqueued
 *     (except TGEMM_ELAUNCH).
 */
#ifndef TGEMM_H_
#define TGEMM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define TGEMM_API __attribute__((visibility("default")))
#else
#define TGEMM_API
#endif

#define TGEMM_OK 0
#define TGEMM_EINVAL_DIM (-1)   /* M, N or K negative, or larger than TGEMM_MAX_DIM, or an  */
                                /* output that needs 2^31 or more workgroups in one launch */
#define TGEMM_EINVAL_LD (-2)    /* lda < max(1,K), ldb < max(1,N), ldc < max(1,N) (with    */
                                /* transposed operands lda < max(1,M), ldb < max(1,K))     */
#define TGEMM_ENULL (-3)        /* NULL pointer for an operand with a nonzero extent        */
#define TGEMM_EDEVICE (-4)      /* current HIP device is not gfx950, or no device           */
#define TGEMM_ELAUNCH (-5)      /* the kernel launch was rejected by the HIP runtime        */
#define TGEMM_EINVAL_CFG (-6)   /* config index out of range, or config not usable here     */
#define TGEMM_EALIGN (-7)       /* A, B or C not aligned to 2 bytes (one binary16 element), */
                                /* or a workspace not aligned to 256 bytes                 */
#define TGEMM_EWORKSPACE (-8)   /* workspace smaller than tgemm_workspace_bytes requires    */

#define TGEMM_MAX_DIM ((int64_t)1 << 31)  /* M, N, K must be < 2^31                        */
/* Any leading dimension at or above the row length is served. The fast kernels address
 * a 256-row operand tile through a 32-bit buffer range, so lda and ldb above
 * TGEMM_FAST_MAX_LD elements (binary16; bytes for fp8 codes: twice that) take the
 * generic kernels, which index in 64 bits. ldc is not limited. */
#define TGEMM_FAST_MAX_LD ((int64_t)1 << 22)

/*
 * C = ReLU(A @ B) if relu != 0, else C = A @ B.
 *   M, N, K   : sizes; M == 0 or N == 0 is a no-op; K == 0 writes C = 0 (the empty sum).
 *   A, lda    : M x K binary16 matrix and its row stride in elements (lda >= max(1, K)).
 *   B, ldb    : K x N binary16 matrix and its row stride (ldb >= max(1, N)).
 *   C, ldc    : M x N binary16 output and its row stride (ldc >= max(1, N)); only the
 *               M x N elements are written, padding between rows is untouched.
 *   relu      : 0 = plain GEMM, any other value = fused ReLU.
 *   stream    : hipStream_t as void*, NULL for the default stream.
 * The fast path needs A, B, C 16-byte aligned, lda, ldb, ldc multiples of 8, lda and
 * ldb at most TGEMM_FAST_MAX_LD, and K, N multiples of 8; other arguments take a slower
 * generic kernel with the same results (within the stated tolerance; both accumulate in
 * float32).
 * Returns TGEMM_OK or a negative TGEMM_E* code.
 */
TGEMM_API int gemm_f16(int64_t M, int64_t N, int64_t K,
             const void* A, int64_t lda,
             const void* B, int64_t ldb,
             void* C, int64_t ldc,
             int relu, void* stream);

/*
 * C = ReLU(op(A) @ op(B)) if relu != 0, else C = op(A) @ op(B), with the operands given
 * either way round -- the transposed-operand GEMMs of the autograd wrapper in
 * "TileLang-MUSA operator development" (7yue.com), section 6, whose backward computes
 * dA = dC @ B^T and dB = A^T @ dC:
 *   trans_a == 0 : op(A) = A, stored M x K row-major, lda >= max(1, K);
 *   trans_a != 0 : op(A) = A^T, A stored K x M row-major, lda >= max(1, M);
 *   trans_b == 0 : op(B) = B, stored K x N row-major, ldb >= max(1, N);
 *   trans_b != 0 : op(B) = B^T, B stored N x K row-major, ldb >= max(1, K).
 * Everything else as gemm_f16 (which is gemm_f16_ex(0, 0, ...)). The fast path needs A, B,
 * C 16-byte aligned, lda, ldb, ldc multiples of 8, lda and ldb at most TGEMM_FAST_MAX_LD,
 * N a multiple of 8 and each operand's contiguous dimension (K for A and for B^T, M for
 * A^T, N for B) a multiple of 8; other arguments take the generic kernel. On the fast path the result is bit-for-bit the same
 * for all four layouts of the same logical operands.
 */
TGEMM_API int gemm_f16_ex(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda,
                          const void* B, int64_t ldb,
                          void* C, int64_t ldc,
                          int relu, void* stream);

/*
 * Split-K for output grids too small to fill the GPU: gemm_f16_ex's operation, computed
 * by `splits` workgroups per output tile, each over a contiguous range of k-tiles, the
 * partial sums combined in a fixed order. This carries the pages' idea of splitting a
 * long reduction across compute units and combining the parts afterwards (the Split-KV
 * decoding of "Writing High-Performance Kernels in TileLang, from GEMM to MLA"
 * (atlascloud.ai), MLA section) over to the GEMM's K.
 *   workspace, workspace_bytes : caller-owned device memory, 256-byte aligned, at least
 *       tgemm_workspace_bytes(trans_a, trans_b, M, N, K) bytes (0 means the call does not
 *       split and the workspace may be NULL). The whole workspace must be zero-filled
 *       before its first use; every call leaves its counter region at zero again, so one
 *       workspace serves any number of calls of any shapes in stream order. Calls that
 *       may overlap in time (different streams) need different workspaces.
 * The library picks the tile config and the split count (tgemm_split_plan shows them);
 * when the output grid fills the GPU it does not split and equals gemm_f16_ex. Results
 * are deterministic: the last split to finish a tile adds the fp32 partial tiles in split
 * order, whichever it is, then applies ReLU and rounds to fp16 once. They differ from the
 * unsplit kernel's only by fp32 summation order (same tolerance).
 * Returns TGEMM_OK, the argument errors of gemm_f16_ex, TGEMM_ENULL (workspace NULL when
 * needed), TGEMM_EALIGN (workspace alignment) or TGEMM_EWORKSPACE.
 */
TGEMM_API int64_t tgemm_workspace_bytes(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K);
TGEMM_API int gemm_f16_ws(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda,
                          const void* B, int64_t ldb,
                          void* C, int64_t ldc,
                          int relu, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The workspace bytes gemm_f16_ws_cfg needs for config idx and split count splits over an
 * M x N output: 0 when splits == 1, else a 4 KiB counter region plus splits fp32 partial
 * tiles per output tile. TGEMM_EINVAL_CFG when gemm_f16_ws_cfg would reject idx or splits
 * for this output, TGEMM_EINVAL_DIM for sizes outside [0, 2^31). Pure host logic.
 */
TGEMM_API int64_t tgemm_workspace_bytes_cfg(int idx, int splits, int64_t M, int64_t N);

/*
 * gemm_f16_ws for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same operation,
 * tile config and split plan, bit for bit the same results, but the split-K scratch (tile
 * counters and fp32 partial tiles) is a static device array of the library instead of a
 * caller workspace. The call allocates nothing and calls no allocating routine.
 *   - The array holds TGEMM_STATIC_SCRATCH_BYTES bytes on every device the library runs
 *     on, from the first use on that device until the process ends. A plan needing more
 *     returns TGEMM_EWORKSPACE before anything is enqueued (the current split plans need
 *     at most 4 KiB + 64 MiB: 256 partial tiles of 256 x 256 floats).
 *   - The counters are zero when the library is loaded and every call leaves them at zero;
 *     the partial tiles keep the last call's contents, which no later call reads before
 *     writing.
 *   - All calls on one device share the array: calls that may overlap in time on one
 *     device (different streams, or different host threads) race and give wrong results.
 *     Order them on one stream.
 *   - The first call on a device looks the array's device address up
 *     (hipGetSymbolAddress); make that first call outside graph capture.
 * Arguments and return codes as gemm_f16_ex, plus TGEMM_EWORKSPACE as above.
 */
#define TGEMM_STATIC_SCRATCH_BYTES ((int64_t)4096 + ((int64_t)64 << 20))
TGEMM_API int gemm_f16_ws_static(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                                 const void* A, int64_t lda,
                                 const void* B, int64_t ldb,
                                 void* C, int64_t ldc,
                                 int relu, void* stream);

/*
 * Grouped GEMM: count independent GEMMs C_i = ReLU?(op(A_i) @ op(B_i)) with one operand
 * layout and one ReLU flag for all, any sizes per GEMM (e.g. the experts of a
 * mixture-of-experts layer, each with its own number of rows: the "MoE GroupGEMM" planned
 * in "TileLang-MUSA operator development" (7yue.com), section 7). GEMMs on the fast path
 * are launched together, up to 32 per launch, with one tile config chosen from their
 * total size; the others (K == 0, or arguments only the generic kernel takes) get a
 * launch of their own; M_i == 0 or N_i == 0 is skipped. gemms: host array of count
 * descriptors (read during the call only). Every descriptor is validated before any work
 * is enqueued; the first invalid one's error code is returned. C_i must not overlap any
 * A_j, B_j or another C_j. Otherwise as gemm_f16_ex.
 */
typedef struct tgemm_gemm_desc {
    int64_t M, N, K;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    void* C;
    int64_t ldc;
} tgemm_gemm_desc;
TGEMM_API int gemm_f16_grouped(int trans_a, int trans_b, int count, const tgemm_gemm_desc* gemms,
                               int relu, void* stream);

/* Human-readable text for a return code (static storage, never NULL). */
TGEMM_API const char* tgemm_strerror(int code);

/* Library version string (static storage). */
TGEMM_API const char* tgemm_version(void);

/* ---- tooling: config table (used by the offline sweep, the benchmark and tests) ---- */

/* Description of one compiled kernel configuration. */
/*
 * fp8 (E4M3) block-scaled GEMM -- the fp8_block_scaled_linear(x, w_fp8, scale_w,
 * block=128) of "TileLang-MUSA operator development" (7yue.com), section 8.2, with the
 * per-block scaling the TileLang write-up measured on A100 (nxmr.cn 138173), section 7,
 * names ("block scaling as in CUTLASS"). The pages fix neither the fp8 encoding nor the
 * block shapes nor the scale type; the reading taken here is the block-scaled recipe those
 * names refer to:
 *   codes      : OCP E4M3 ("E4M3FN"): 1 sign, 4 exponent bits (bias 7), 3 fraction bits,
 *                no infinities, S.1111.111 = NaN, largest finite 448;
 *   A, lda     : M x K codes (one byte each), row-major with k contiguous (activations),
 *                lda in bytes >= max(1, K);
 *   scale_a    : M x KB float32, contiguous (row i at scale_a + i * KB), KB = ceil(K/128):
 *                one scale per 1 x 128 block of A;
 *   B, ldb     : N x K codes, row-major with k contiguous (a linear layer's weight, out x
 *                in features), ldb >= max(1, K);
 *   scale_b    : ceil(N/128) x KB float32, contiguous: one scale per 128 x 128 block of B;
 *   C, ldc     : M x N binary16 output (round to nearest even), ldc >= max(1, N);
 *   C[i,j] = ReLU?( sum_kb scale_a[i,kb] * scale_b[j/128,kb] * sum_{k in kb} a[i,k] * b[j,k] )
 * where block kb holds k in [128 kb, min(K, 128 kb + 128)). On the fast path each block's
 * 128 products are summed by the fp8 matrix instructions (exact products; their block sum
 * may deviate from the exact one by up to about 2^-10 of the block's largest product) and
 * the scaled block sums are accumulated in float32 -- the per-block promotion the scaling
 * is for. The fast path needs A and B 16-byte aligned, lda, ldb and K multiples of 16,
 * lda and ldb at most 2 * TGEMM_FAST_MAX_LD bytes, C 16-byte aligned and ldc, N multiples
 * of 8; other arguments take a generic kernel that sums each block in float32. M == 0 or N == 0 is a no-op, K == 0 writes C = 0. Device
 * pointers, ownership, streams and errors as for gemm_f16; scale_a and scale_b must be
 * 4-byte aligned (else TGEMM_EALIGN) and, when K > 0, non-NULL (else TGEMM_ENULL).
 */
TGEMM_API int gemm_fp8_block(int64_t M, int64_t N, int64_t K,
                             const void* A, int64_t lda, const float* scale_a,
                             const void* B, int64_t ldb, const float* scale_b,
                             void* C, int64_t ldc, int relu, void* stream);

/*
 * Block quantizer to E4M3 for gemm_fp8_block (the step that brings x to fp8 inside
 * fp8_block_scaled_linear; the same reading as above). X: R x K binary16 (ldx elements);
 * Q: R x K codes (ldq bytes, both >= max(1, K)); scale: ceil(R/block_rows) x KB float32,
 * contiguous. block_rows = 1 quantizes per 1 x 128 block (activations, scale_a), 128 per
 * 128 x 128 block (weights, scale_b); any other value is TGEMM_EINVAL_DIM. For a block
 * whose largest magnitude is amax (float32): s = amax / 448 in float32 (s = 1 for an
 * all-zero block), q = E4M3(x / s) with float32 division rounded to nearest, then rounded
 * to nearest even and saturated to +-448. Finite inputs only (NaN or infinity in a block
 * gives unspecified codes and scale). R == 0 or K == 0 is a no-op. X must be 2-byte and
 * scale 4-byte aligned; 16-byte aligned X, 8-byte aligned Q and ldx, ldq, K multiples of 8
 * take vector loads and stores. Otherwise as gemm_f16.
 */
TGEMM_API int quant_fp8_block(int64_t R, int64_t K, const void* X, int64_t ldx, int block_rows,
                              void* Q, int64_t ldq, float* scale, void* stream);

typedef struct tgemm_config_info {
    int32_t block_m, block_n, block_k; /* workgroup tile (elements)                     */
    int32_t stages;                    /* LDS pipeline depth                            */
    int32_t waves_m, waves_n;          /* wavefront grid inside the workgroup           */
    int32_t panel;                     /* tile-rows per panel of the workgroup order    */
    int32_t xcd_remap;                 /* 1 = consecutive tiles kept on one XCD         */
    int32_t generic;                   /* 1 = unaligned-capable generic kernel          */
    int32_t lds_bytes;                 /* dynamic LDS per workgroup                     */
    int32_t layouts;                   /* bit (2*trans_a + trans_b) set: layout accepted */
    int32_t built;                     /* 1 = compiled into this library; 0 = a tooling  */
                                       /* variant only the tooling build compiles (the   */
                                       /* _cfg entry points refuse it here)              */
    char name[48];
} tgemm_config_info;

/* Number of configurations in the table. */
TGEMM_API int tgemm_num_configs(void);

/* Fills *out for config idx; returns TGEMM_OK or TGEMM_EINVAL_CFG / TGEMM_ENULL. */
TGEMM_API int tgemm_config_desc(int idx, tgemm_config_info* out);

/* Index of the config gemm_f16 would use for these arguments (pure host logic, no HIP
 * call). Returns a negative TGEMM_E* code for invalid arguments, or -100 when the call
 * launches nothing (M == 0 or N == 0) and -101 when it only zero-fills C (K == 0). */
TGEMM_API int tgemm_select_config(int64_t M, int64_t N, int64_t K,
                        const void* A, int64_t lda,
                        const void* B, int64_t ldb,
                        const void* C, int64_t ldc);

/* tgemm_select_config for gemm_f16_ex's operand layouts. */
TGEMM_API int tgemm_select_config_ex(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                        const void* A, int64_t lda,
                        const void* B, int64_t ldb,
                        const void* C, int64_t ldc);

/* gemm_f16_ex forced to config idx (TGEMM_EINVAL_CFG also when the config does not take
 * this operand layout, see tgemm_config_info.layouts). */
TGEMM_API int gemm_f16_ex_cfg(int idx, int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda,
                  const void* B, int64_t ldb,
                  void* C, int64_t ldc,
                  int relu, void* stream);

/* The plan gemm_f16_ws would use for these arguments: config index, split count (1 = no
 * split) and the workspace bytes it needs. Pure host logic. Returns TGEMM_OK, TGEMM_ENULL
 * for a NULL output pointer or an argument error of gemm_f16_ex. */
TGEMM_API int tgemm_split_plan(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda,
                  const void* B, int64_t ldb,
                  const void* C, int64_t ldc,
                  int* cfg, int* splits, int64_t* workspace_bytes);

/* gemm_f16_ws forced to config idx and split count splits (1 .. 8; > 1 only for configs
 * taking all four layouts, at most ceil(K / block_k) splits and 1024 output tiles;
 * otherwise TGEMM_EINVAL_CFG). */
TGEMM_API int gemm_f16_ws_cfg(int idx, int splits, int trans_a, int trans_b,
                  int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda,
                  const void* B, int64_t ldb,
                  void* C, int64_t ldc,
                  int relu, void* workspace, int64_t workspace_bytes, void* stream);

/* gemm_f16 forced to config idx (same arguments and error codes; TGEMM_EINVAL_CFG if
 * idx is out of range or the fast config cannot take these pointers / strides). */
TGEMM_API int gemm_f16_cfg(int idx, int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 void* C, int64_t ldc,
                 int relu, void* stream);

/* Host replica of the device's workgroup -> output-tile map of config idx (the same
 * inline function the kernels run): for workgroup id wg of a launch over an M x N
 * output, writes the tile coordinates (*tile_m, *tile_n). Returns TGEMM_OK,
 * TGEMM_EINVAL_CFG, TGEMM_ENULL, or TGEMM_EINVAL_DIM if wg is outside the launch or M
 * or N is outside 1 .. TGEMM_MAX_DIM - 1. */
TGEMM_API int tgemm_tile_of(int idx, int64_t M, int64_t N, int64_t wg,
                  int64_t* tile_m, int64_t* tile_n);

/* The same map for a split-K launch of config idx with `splits` splits per tile
 * (tiles x splits workgroups; splits = 1 gives tgemm_tile_of's map): writes the tile
 * and the split (0 .. splits - 1) workgroup wg computes. Returns TGEMM_OK,
 * TGEMM_EINVAL_CFG (idx out of range, splits outside 1 .. 8, or splits > 1 for a config
 * that cannot split), TGEMM_ENULL, or TGEMM_EINVAL_DIM as for tgemm_tile_of. */
TGEMM_API int tgemm_split_tile_of(int idx, int64_t M, int64_t N, int splits, int64_t wg,
                        int64_t* tile_m, int64_t* tile_n, int* split);

/* Number of workgroups config idx launches for an M x N output (-1 for an idx out of
 * range, or M or N outside 0 .. TGEMM_MAX_DIM - 1). */
TGEMM_API int64_t tgemm_num_workgroups(int idx, int64_t M, int64_t N);


/* fp8 tooling: the fp8 tile configs (tgemm_config_info with block_k = 128 and layouts =
 * 2: A as given, B transposed), the config gemm_fp8_block would pick (scales not looked
 * at; TGEMM_FP8_GENERIC for the generic kernel, -100 / -101 as for tgemm_select_config),
 * and gemm_fp8_block forced onto config idx (or TGEMM_FP8_GENERIC; TGEMM_EINVAL_CFG if a
 * fast config cannot take the arguments). */
#define TGEMM_FP8_GENERIC (-102)
TGEMM_API int tgemm_fp8_num_configs(void);
TGEMM_API int tgemm_fp8_config_desc(int idx, tgemm_config_info* out);
TGEMM_API int tgemm_fp8_select_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                      const void* B, int64_t ldb, const void* C, int64_t ldc);
TGEMM_API int gemm_fp8_block_cfg(int idx, int64_t M, int64_t N, int64_t K,
                                 const void* A, int64_t lda, const float* scale_a,
                                 const void* B, int64_t ldb, const float* scale_b,
                                 void* C, int64_t ldc, int relu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H_ */
