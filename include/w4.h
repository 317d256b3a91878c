/*
 * w4.h -- C ABI of the MI355X (gfx950) fused 4-bit weight-only dequantize-and-multiply library.
 *
 * The operation: y[b, n] = sum_k x[b, k] * W_hat[n, k], where W_hat is decoded on chip from packed
 * 4-bit weights and per-block scales, with fp32 accumulation, and never written back to memory
 * (LLM Quantization on RTX 4060: Where 4-bit Decode Falls Behind FP16, sections "Fused Kernel:
 * Moving Dequantization On-Chip" and "Kernel Implementation").
 *
 * Conventions shared by every entry point
 *   - Every pointer named as "device" is HIP device memory owned by the caller; the library never
 *     allocates, frees or keeps a device pointer beyond the call.
 *   - All arrays are dense and row-major; there are no stride arguments.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Matmul calls are
 *     asynchronous on it and make no allocation and no synchronization, so they can be captured
 *     in a HIP graph.  Quantize calls synchronize the stream (they report device-detected errors).
 *   - Arguments are validated on the host before anything is launched; a failing check returns a
 *     negative w4_status_t and launches nothing.  After a launch, a HIP launch error is reported
 *     as W4_ERR_HIP.
 *   - Packed weights: uint8 [N, K/2]; byte i of a row holds element 2i in its high nibble and
 *     element 2i+1 in its low nibble (same page, "Kernel Implementation").
 *   - Library state (everything that outlives a call):
 *       . a path override and one registered workspace per device (w4_set_path, w4_set_workspace,
 *         and the environment variable W4_FORCE_PATH, read once when the library is loaded); they
 *         steer only w4_gemv and w4_gemm_smallbatch and are read under a lock at each call;
 *       . one device-side non-finite flag word for the quantizers and one for the 2:4 compression
 *         (per device); a call resets its word, launches, synchronizes and reads it back under a
 *         host lock, so concurrent quantize or compress calls are serialized by the library;
 *       . a helper stream and two events per device for w4_gptq_quantize on large layers,
 *         created on first use and kept until the process ends;
 *       . a cache of each device's compute-unit count (launch shapes);
 *       . the split-K scratch of w4_matmul_splitk_noalloc: a static device array per device and
 *         its looked-up address per device.
 *     Matmul calls on different streams may run concurrently as long as their buffers (and
 *     workspaces) do not overlap.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight format x activation dtype.  y is always fp32 [B, N].
 *   NF4 : 16-entry NormalFloat codebook, blocks of 64 along K, one fp32 absmax per block,
 *         scales = float[N, K/64]  (LLM Quantization on RTX 4060, "Standard Expectation from
 *         Quantization").
 *   INT4: symmetric, stored nibble = q + 8 (My Triton Kernel Ties bitsandbytes, "The kernels"),
 *         groups of 128 along K, scales = bf16 bit patterns uint16[N, K/128].
 *   FP4 : E2M1 codes through a 16-entry table (nibble bit 3 = sign, bits 0-2 index the
 *         magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; LLM Compressor 0.14, "Details worth
 *         knowing"), blocks of 64 along K, one fp32 scale absmax / 6 per block,
 *         scales = float[N, K/64]; decoded weight = table[nibble] * scale.
 *   INT4A: asymmetric INT4 (LLM Compressor 0.14, "The fused kernel": a code is the scale
 *         quotient plus the zero point, clamped and rounded; "What those numbers leave out":
 *         INT4 in symmetric and asymmetric grouped forms): nibble = unsigned code q in 0..15, groups of 128 along K,
 *         scales = uint32[N, K/128] words, bf16 scale bits in bits 0-15 and the zero point z
 *         (0..15) in bits 16-19, bits 20-31 zero; decoded weight = (q - z) * scale. */
typedef enum {
  W4_NF4_X_F16 = 1,
  W4_NF4_X_BF16 = 2,
  W4_INT4_X_F16 = 3,
  W4_INT4_X_BF16 = 4,
  W4_FP4_X_F16 = 5,
  W4_FP4_X_BF16 = 6,
  W4_INT4A_X_F16 = 7,
  W4_INT4A_X_BF16 = 8
} w4_format_t;

typedef enum {
  W4_OK = 0,
  W4_ERR_NULL = -1,      /* a required pointer is NULL                                        */
  W4_ERR_SHAPE = -2,     /* N, K or B out of range, or K not a multiple of 64 (NF4, FP4) / 128 (INT4, INT4A) */
  W4_ERR_ALIGN = -3,     /* packed or x not 16-byte aligned, scales or y not element aligned  */
  W4_ERR_FORMAT = -4,    /* unknown w4_format_t                                               */
  W4_ERR_NONFINITE = -5, /* quantize met a NaN or Inf weight (outputs are then meaningless)   */
  W4_ERR_WORKSPACE = -6, /* workspace missing or smaller than w4_workspace_bytes()            */
  W4_ERR_PATH = -7,      /* unknown path, or a path that does not support this batch size     */
  W4_ERR_HIP = -8,       /* a HIP runtime call failed                                         */
  W4_ERR_ALIAS = -9      /* y overlaps an input or the workspace                              */
} w4_status_t;

/* Execution paths of the matmul. */
typedef enum {
  W4_PATH_AUTO = 0,    /* pick by (format, N, K, B) from a fixed table                        */
  W4_PATH_GEMV = 1,    /* fused streaming GEMV, one pass, B <= 8                              */
  W4_PATH_SPLITK = 2,  /* fused GEMV over split_k disjoint K ranges into an fp32 workspace,
                          then a fixed-order sum that overwrites y (deterministic, no atomics;
                          My Triton Kernel Ties bitsandbytes, "The kernels", v3 and its
                          stale-output bug)                                                  */
  W4_PATH_MFMA = 3,    /* decode W on chip, MFMA against x, 1 <= B <= W4_MAX_BATCH (W4_PATH_AUTO
                          takes it from B = 4; from B = 3 for matrices of 64 MiB and more,
                          from B = 5 for matrices under 4 MiB).
                          With split_k >= 2: K in split_k ranges of whole 256-weight quads
                          (fewer when the quads do not fill them), each range's partial sums
                          into an fp32 workspace, then the same fixed-order sum as
                          W4_PATH_SPLITK; W4_PATH_AUTO splits rows longer than 3072 weights
                          when the workspace holds the partials                              */
  W4_PATH_TWOPASS = 4, /* ablation: dequantize W to fp16 in the workspace, then a dense GEMV/GEMM
                          (the out-of-place path of LLM Quantization on RTX 4060, "The
                          Quantization Tax: A Byte-Accounting Model")                        */
  W4_PATH_TILED = 5,   /* prefill-size GEMM: output tiles of 128 weight rows x 128 activation
                          rows, K walked one 64-weight block at a time, weights decoded on chip
                          into the matrix-core operands (LLM Quantization on RTX 4060, "Why Only
                          16%", item 3: prefill needs a GEMM, not a GEMV per token); any B.
                          W4_PATH_AUTO takes it from B = W4_TILED_FROM_BATCH for matrices of
                          N >= W4_TILED_FROM_ROWS, and for fewer rows when K splits (below) and
                          the workspace holds the partials (else the MFMA path is faster there).
                          With split_k >= 2 K runs in ranges of whole 64-weight blocks on
                          separate workgroups, partial sums in the workspace, then the fixed-order
                          reduction; W4_PATH_AUTO, given a workspace, splits K into the smallest
                          power of two of ranges that gives three quarters of the CUs a 64-row
                          tile, each range at least 16 blocks, at most 16 ranges.  For fp16
                          activations (W4_NF4_X_F16, W4_INT4_X_F16, W4_FP4_X_F16,
                          W4_INT4A_X_F16) from 128
                          activation rows the folded kernel of W4_PATH_TILED_F16 runs instead
                          where its rules take it (see there), with that kernel's split rule for
                          W4_PATH_AUTO                                                          */
  W4_PATH_TILED_F16 = 6 /* prefill-size GEMM for fp16 activations with each block scale folded into
                          the decoded fp16 weights (one packed multiply per weight pair), so the
                          matrix cores accumulate x * W_hat over all of K: tiles of 256 or 128
                          weight rows x 128 activation rows, 32x32x16 matrix steps; any B; no
                          workspace in one pass (split_k <= 1), else K in ranges of whole
                          64-weight blocks (128-row tiles; an even number of blocks per range
                          for INT4 and asymmetric INT4), partial sums in the workspace, the
                          fixed-order reduction.  W4_NF4_X_F16, W4_INT4_X_F16, W4_FP4_X_F16 and
                          W4_INT4A_X_F16 only (other formats: W4_ERR_PATH).  A folded weight is
                          within 3 * 2^-11 of W_hat (NF4; FP4 2 * 2^-11; asymmetric INT4 2^-11;
                          INT4 exact); a wave whose
                          rows hold a block scale outside the range where every folded weight is a
                          normal, finite fp16 number (NF4 [2^-10, 2^15], FP4 [2^-13, 2^13], INT4
                          and asymmetric INT4 [2^-14, 2^12], or zero) runs all of K with the
                          scale applied in fp32 per
                          block instead.  W4_PATH_AUTO and W4_PATH_TILED take it for those
                          formats from 128 activation rows: in one pass over 128 weight rows
                          by 192 activation rows per tile when 128 < B <= 192 and the matrix
                          has at least 128 weight rows per CU; else with 256-row tiles when
                          B > 128 and those number at least two per CU (one per CU for
                          K >= 4096), else with 128-row tiles when those number at least one per
                          CU (half a tile per CU when B > 128 and K < 4096); split launches from
                          256 rows, and from 128 with at least 32 tiles of 128 rows.
                          W4_PATH_AUTO with a workspace splits K for it when its T 128-row tiles
                          number under one per CU and K >= 4096 (below 256 rows: T >= 32): into
                          min(16, 2 CUs / T) ranges when each keeps at least 32 blocks of 64
                          weights, else min(16, CUs / T, K / 64 / 12) (at least 2 when
                          T >= CUs / 2) if that is at least 2; and into two ranges when
                          1 <= T / CUs < 2 and K >= 16384                                       */
} w4_path_t;

#define W4_MAX_BATCH 4096
#define W4_TILED_FROM_BATCH 128
#define W4_TILED_FROM_ROWS 4096
#define W4_MAX_SPLIT_K 64
#define W4_MAX_GROUP 4
#define W4_NOALLOC_SCRATCH_BYTES (8 << 20) /* static split-K scratch of w4_matmul_splitk_noalloc */

/* ---------------------------------------------------------------- quantizers (offline) ----- */

/* w4_quantize_nf4: blockwise absmax NF4 (LLM Quantization on RTX 4060, "Standard Expectation
 * from Quantization").  Per row and 64-block: absmax A = max |w| (stored as fp32, not re-
 * quantized); nibble = index of the code nearest to w / A, decided exactly (fp64 quotient
 * against fp64 midpoints; a value exactly on a midpoint takes the lower index); a block with
 * A == 0 stores A = 0 and nibble 7 (the 0.0 code).
 *   w       device float[N, K], read only
 *   N, K    N >= 1, K >= 64, K % 64 == 0
 *   packed  device uint8[N, K/2], written; 16-byte aligned
 *   absmax  device float[N, K/64], written; 4-byte aligned
 * Synchronizes `stream`.  Returns W4_ERR_NONFINITE if any weight is NaN or Inf. */
int w4_quantize_nf4(const float* w, int64_t N, int64_t K, uint8_t* packed, float* absmax,
                    void* stream);

/* w4_quantize_int4: symmetric INT4 with a +8 zero point (My Triton Kernel Ties bitsandbytes,
 * "The kernels"), round half to even (LLM Compressor 0.14, "Details worth knowing").  Per row and
 * 128-group: s = bf16_RNE(fp32(absmax / 7)); q = clamp(rint(w / s), -8, 7) with the quotient
 * taken against the rounded s; nibble = q + 8; a group whose s is 0 stores s = 0, nibbles 8.
 *   w           device float[N, K], read only
 *   N, K        N >= 1, K >= 128, K % 128 == 0
 *   packed      device uint8[N, K/2], written; 16-byte aligned
 *   scale_bf16  device uint16[N, K/128] (bf16 bit patterns), written; 2-byte aligned
 * Synchronizes `stream`.  Returns W4_ERR_NONFINITE if any weight is NaN or Inf. */
int w4_quantize_int4(const float* w, int64_t N, int64_t K, uint8_t* packed, uint16_t* scale_bf16,
                     void* stream);

/* w4_quantize_int4_asym: asymmetric INT4 (LLM Compressor 0.14, "The fused kernel": a code is the
 * weight divided by the scale, plus the zero point, clamped and rounded; "Details worth knowing":
 * rint).  Per row and 128-group: lo = min(min w, 0), hi = max(max w, 0);
 * s = bf16_RNE(fp32(fp32(hi - lo) / 15)); z = clamp(rint(-lo / s), 0, 15);
 * q = rint(clamp(w / s + z, 0, 15)), the quotients in fp64 against the rounded s; a group whose
 * s is 0 stores word 0 and nibbles 0.
 *   w       device float[N, K], read only; 8-byte aligned
 *   N, K    N >= 1, K >= 128, K % 128 == 0
 *   packed  device uint8[N, K/2], written; 16-byte aligned; element 2i in the high nibble
 *   words   device uint32[N, K/128], written: bf16 bits of s | z << 16; 4-byte aligned
 * Synchronizes `stream`.  Returns W4_ERR_NONFINITE if any weight is NaN or Inf. */
int w4_quantize_int4_asym(const float* w, int64_t N, int64_t K, uint8_t* packed, uint32_t* words,
                          void* stream);

/* w4_quantize_fp4: FP4 (E2M1) quantization, blocks of 64 along K (LLM Compressor 0.14: GPTQ's 15x
 * speedup is one fused loop, "Details worth knowing": threshold comparisons onto
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} whose <= and < alternate, so exact ties land on even codes).
 *   w      device float[N, K] (fp32), read only; 8-byte aligned
 *   N, K   N >= 1, K a positive multiple of 64
 *   packed device uint8[N, K/2], written; 16-byte aligned; element 2i in the high nibble
 *   scale  device float[N, K/64], written: s = fp32(absmax / 6) of each block (0 for an all-zero
 *          block, whose nibbles are all 0); 4-byte aligned
 * Nibble of w: sign bit (w < 0) | ladder index of |w| / s, the quotient taken in fp64.
 * Synchronizes `stream`.  Returns W4_ERR_NONFINITE if any weight is NaN or Inf. */
int w4_quantize_fp4(const float* w, int64_t N, int64_t K, uint8_t* packed, float* scale,
                    void* stream);

/* -------------------------------------------------------------------------- matmul --------- */

/* ---------------------------------------------------------------- settings ----------------- */

/* w4_set_path: a path override for the automatic choice of w4_gemv and w4_gemm_smallbatch (the
 * wrapper's checks of LLM Quantization on RTX 4060, "Kernel Implementation", turned into a knob
 * for tests and ablations; My Triton Kernel Ties bitsandbytes, "The kernels", bug 2: compare paths
 * explicitly rather than trusting an automatic pick).  path = W4_PATH_AUTO removes the override.
 * While an override is set, those two calls run w4_matmul_ex with that path, split_k = 0 and the
 * workspace registered for the current device; a path that cannot run the arguments returns
 * W4_ERR_PATH, a split-K or two-pass override without a large enough registered workspace returns
 * W4_ERR_WORKSPACE.  Other entry points ignore the override.  The environment variable
 * W4_FORCE_PATH (auto, gemv, splitk, mfma, twopass, tiled, tiled_f16, or the digit 0-6) sets the same
 * override once, when the library is loaded; an unknown value makes the steered calls return
 * W4_ERR_PATH until w4_set_path is called.  Process-wide, not per thread: set it before launching
 * work from other threads.  Returns W4_OK, or W4_ERR_PATH for an unknown path.  Host only; no
 * allocation, no device call. */
int w4_set_path(int path);

/* The current override (a w4_path_t), or W4_ERR_PATH when W4_FORCE_PATH held an unknown value. */
int w4_get_path(void);

/* w4_set_workspace: registers caller-owned device memory for the current device, used by w4_gemv
 * and w4_gemm_smallbatch when a path needs scratch (split-K partials, two-pass decoded weights).
 *   workspace  device memory, 16-byte aligned, or NULL with bytes = 0 to unregister
 *   bytes      its size
 * The library keeps the pointer (it never frees it); the caller keeps the memory alive and unused
 * by anything else while steered calls may run, and calls that share it must not overlap in time.
 * Returns W4_OK, W4_ERR_NULL (NULL with bytes > 0), W4_ERR_ALIGN or W4_ERR_HIP (no current device).
 * Host only; no allocation. */
int w4_set_workspace(void* workspace, size_t bytes);

/* ---------------------------------------------------------------- matmul ------------------- */

/* w4_gemv: fused dequantize-and-multiply, y = x . W_hat^T, B <= 8 (decode; LLM Quantization on
 * RTX 4060, "Kernel Implementation": unpack, codebook, block scale, fp32 accumulation).
 *   x       device [B, K] fp16 or bf16 (per fmt) bit patterns; 16-byte aligned
 *   packed  device uint8[N, K/2]; 16-byte aligned
 *   scales  device float[N, K/64] (NF4) or uint16 bf16 bits [N, K/128] (INT4)
 *   fmt     w4_format_t
 *   N, K, B N >= 1; K as for the format; 1 <= B <= 8
 *   y       device float[B, N]; fully overwritten, never accumulated into; must not overlap inputs
 * Single pass, no workspace (unless w4_set_path steers it to another path).  Asynchronous on
 * `stream`. */
int w4_gemv(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t N,
            int64_t K, int64_t B, float* y, void* stream);

/* w4_gemv_grouped: G weight matrices that read the same activations (a layer's q, k and v
 * projections, or its gate and up projections) in ONE launch of the fused GEMV:
 * y_g = x . W_hat_g^T for g = 0 .. G-1.  Stacking modules that share their input so that one
 * launch covers them gives fewer, fuller launches (LLM Compressor 0.14: GPTQ's 15x speedup is one
 * fused loop, section "Batching layers"); at decode sizes the launch itself is a large share of a
 * small GEMV's time (My Triton Kernel Ties bitsandbytes, "The numbers" and "What's next").
 *   x        device [B, K] fp16 or bf16 bit patterns, shared by every member; 16-byte aligned
 *   groups   G, 1 <= G <= W4_MAX_GROUP
 *   packed   host array of G device pointers, member g: uint8[N_g, K/2]; 16-byte aligned
 *   scales   host array of G device pointers, member g: as for w4_gemv with N = N_g
 *   N        host array of G row counts, N_g >= 1, sum of N_g < 2^31
 *   y        host array of G device pointers, member g: float[B, N_g], fully overwritten; no y_g
 *            may overlap another y_h or any input
 *   fmt, K, B  as for w4_gemv, shared by every member (B <= 8)
 * The host arrays are read during the call only.  Each y_g satisfies the same accuracy bound as
 * w4_gemv on that member alone, and is bitwise equal to it when both calls get the same launch
 * shape (w4_gemv_plan with N = N_g and with N = sum of N_g report the same threads, team and
 * iters).  When the fused GEMV has no launch shape for (K, B) (B = 8 with rows of more than 8192
 * values), the members run in one launch of the MFMA kernel instead.  No workspace.
 * Asynchronous on `stream`. */
int w4_gemv_grouped(const void* x, int groups, const uint8_t* const* packed,
                    const void* const* scales, const int64_t* N, float* const* y, int fmt,
                    int64_t K, int64_t B, void* stream);

/* w4_gemm_smallbatch: the same operation for 1 <= B <= W4_MAX_BATCH (decode batches; Do
 * Quantization and Sparsity make LLM Inference Faster?, "NF4: fast at batch 1, slower at larger
 * batches").  Picks the fused GEMV for small B, the MFMA path (weights decoded on chip into
 * the matrix-core operands) for larger B, and the tiled GEMM from B = W4_TILED_FROM_BATCH when
 * N >= W4_TILED_FROM_ROWS; never materializes W_hat.  Arguments as for w4_gemv, with 1 <= B <= W4_MAX_BATCH.
 * No workspace unless one is registered (w4_set_workspace) and a path that needs it is chosen
 * or forced (w4_set_path).  Asynchronous. */
int w4_gemm_smallbatch(const void* x, const uint8_t* packed, const void* scales, int fmt,
                       int64_t N, int64_t K, int64_t B, float* y, void* stream);

/* w4_gemm_prefill: the same operation through the tiled GEMM (W4_PATH_TILED) whatever B: the
 * prompt of a prefill step, B = tokens (LLM Quantization on RTX 4060, "Why Only 16%", item 3).
 *   x       device [B, K] fp16 or bf16 bit patterns, row-major; 16-byte aligned
 *   packed, scales, fmt, N, K, y   as for w4_gemv
 *   B       1 <= B <= W4_MAX_BATCH
 * Returns W4_ERR_PATH when K is 2^22 or more (32-bit offsets inside one tile).  y[b, n] meets the
 * same accuracy bound as w4_gemv.  No workspace.  Asynchronous on `stream`. */
int w4_gemm_prefill(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t N,
                    int64_t K, int64_t B, float* y, void* stream);

/* w4_gemm_smallbatch_grouped: w4_gemv_grouped for 1 <= B <= W4_MAX_BATCH.  The members run in ONE
 * launch of the kernel w4_gemm_smallbatch would pick for a matrix of sum-of-N_g rows: the fused
 * GEMV (as w4_gemv_grouped) for small B, the MFMA kernel over the row tiles of every member for
 * larger B (LLM Compressor 0.14: GPTQ's 15x speedup is one fused loop, section "Batching
 * layers").  From B = W4_TILED_FROM_BATCH the members of N_g >= W4_TILED_FROM_ROWS share one
 * tiled-GEMM launch (their tiles one after another; each y_g is bitwise equal to w4_gemm_prefill
 * on that member when both launches run the same number of K groups per tile: one when a launch
 * has at least two 64 x 128 tiles per CU, two below) and the others share one MFMA launch.  Arguments, ownership and errors as for w4_gemv_grouped, with B up to
 * W4_MAX_BATCH.  Each y_g meets w4_gemm_smallbatch's accuracy bound on that member.  No
 * workspace.  Asynchronous on `stream`. */
int w4_gemm_smallbatch_grouped(const void* x, int groups, const uint8_t* const* packed,
                               const void* const* scales, const int64_t* N, float* const* y,
                               int fmt, int64_t K, int64_t B, void* stream);

/* w4_matmul_ex: the same operation with an explicit path, split count and workspace (tests and
 * the ablation benchmark).  path = W4_PATH_AUTO also considers split-K (fused GEMV, MFMA or tiled
 * GEMM) when a workspace is given: w4_workspace_bytes(..., W4_PATH_AUTO, 0) is the size that lets
 * it.
 * The bytes a path writes into the workspace must not overlap x, packed, scales or y
 * (W4_ERR_ALIAS).
 *   split_k          number of K ranges for W4_PATH_SPLITK (2..W4_MAX_SPLIT_K; 0 = 4), for
 *                    W4_PATH_MFMA, W4_PATH_TILED and W4_PATH_TILED_F16 (2..W4_MAX_SPLIT_K; 0 or
 *                    1 = one pass); ignored by the other paths.  The GEMV and MFMA splits need
 *                    4 * split_k * B * N workspace bytes; the tiled GEMM makes
 *                    R = ceil(K/64 / ceil(K/64 / split_k)) ranges of whole 64-weight blocks
 *                    (R <= split_k) and needs 4 * R * B * N (the folded kernel rounds the blocks
 *                    per range up to an even count for W4_INT4_X_F16, which never adds ranges).
 *   workspace        device memory of at least w4_workspace_bytes(...) bytes, 16-byte aligned;
 *                    may be NULL when that size is 0.  Its contents are scratch on entry and exit.
 *                    Two calls in flight must not share one workspace.
 * Returns W4_ERR_WORKSPACE when the workspace is missing or too small for the requested path. */
int w4_matmul_ex(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t N,
                 int64_t K, int64_t B, float* y, int path, int split_k, void* workspace,
                 size_t workspace_bytes, void* stream);

/* w4_matmul_splitk_noalloc: w4_matmul_ex with path = W4_PATH_SPLITK, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the split-K partials go to a static device array of W4_NOALLOC_SCRATCH_BYTES held by the library
 * on each device it runs on (until the process ends) instead of a caller's workspace.  Same
 * kernels, hence the same bits as w4_matmul_ex with the same split_k.
 *   x, packed, scales, fmt, N, K, B, y   as for w4_gemv (B <= 8)
 *   split_k  2..W4_MAX_SPLIT_K (at most K/32); 0 = 4
 * Returns W4_ERR_WORKSPACE when 4 * split_k * B * N bytes exceed W4_NOALLOC_SCRATCH_BYTES,
 * W4_ERR_PATH for a split count or batch the split-K path cannot run, W4_ERR_HIP when the scratch
 * address cannot be looked up (first call on a device).  Calls no allocating routine.  The scratch
 * is fully rewritten by each call before it is read (nothing needs clearing), but every call on
 * one device shares it: two such calls that overlap in time on one device (two streams, two
 * threads) race and may corrupt each other's y.  Asynchronous on `stream`. */
int w4_matmul_splitk_noalloc(const void* x, const uint8_t* packed, const void* scales, int fmt,
                             int64_t N, int64_t K, int64_t B, float* y, int split_k, void* stream);

/* Bytes of workspace w4_matmul_ex needs for (fmt, N, K, B, path, split_k): split-K (the GEMV's,
 * or the MFMA path's with split_k >= 2) needs 4 * S * B * N, the tiled GEMM's 4 * R * B * N (R its
 * ranges, see w4_matmul_ex), two-pass 2 * N * K, the single-pass paths 0; W4_PATH_AUTO reports the
 * split-K size it would use given that much workspace.
 * Returns 0 for invalid arguments. */
size_t w4_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t B, int path, int split_k);

/* The path (w4_path_t) and split count W4_PATH_AUTO would run for these arguments when given
 * `workspace_bytes` of workspace; negative w4_status_t on invalid arguments. */
int w4_auto_path(int fmt, int64_t N, int64_t K, int64_t B, size_t workspace_bytes, int* split_k);

/* ------------------------------------------------------------------ introspection --------- */

/* Launch shape the fused GEMV uses for (fmt, N, K, B) over `split_k` K ranges (1 = single pass):
 * threads per workgroup, lanes per output row, 16-byte chunks per lane, chunks per split and
 * workgroups along N.  Any output pointer may be NULL.  Returns W4_OK, or W4_ERR_SHAPE /
 * W4_ERR_PATH when the GEMV path cannot run these arguments. */
int w4_gemv_plan(int fmt, int64_t N, int64_t K, int64_t B, int split_k, int* threads, int* team,
                 int* iters, int* chunks_per_split, int* grid_x);

/* Launch shape of w4_gemv_grouped for members of N[0 .. groups-1] rows sharing (fmt, K, B):
 * threads per workgroup, lanes per output row, 16-byte chunks per lane, workgroups along N for all
 * members together (grid_x: each member gets a consecutive range, its share of the grid, at most
 * one workgroup per row block of its own) and grid_z (always 1).  Any output pointer may be NULL.
 * Returns W4_OK, or W4_ERR_SHAPE / W4_ERR_PATH when the grouped GEMV cannot run these arguments
 * (w4_gemv_grouped then runs the members in one launch of the MFMA kernel). */
int w4_gemv_grouped_plan(int fmt, int groups, const int64_t* N, int64_t K, int64_t B, int* threads,
                         int* team, int* iters, int* grid_x, int* grid_z);

/* Host pointer to the 16 NF4 code points (fp32, ascending) the kernels decode with.  Static
 * storage owned by the library; never NULL. */
const float* w4_nf4_codebook(void);

/* Static, human-readable text for a w4_status_t; never NULL. */
const char* w4_status_string(int status);

/* Library ABI version (this header: 1). */
int w4_version(void);

/* ------------------------------------------------------------------ GPTQ column loop ------- */

/* GPTQ quantizes a layer W [rows x cols] column by column onto a grid fixed beforehand, feeding
 * each column's rounding error forward through U, the upper Cholesky factor of the dampened
 * inverse Hessian (H^-1 = U^T U), in lazy blocks of up to 128 columns (LLM Compressor 0.14: GPTQ's
 * 15x speedup is one fused loop, "Three changes that make it fast", "The fused kernel").  Forming
 * H, dampening it and factorizing stay outside these calls, as on that page: U is an input.
 *
 * Common arguments (all device pointers, row-major, 4-byte aligned unless stated):
 *   w       float[rows, cols], read and updated in place: column j ends holding the value it was
 *           quantized from (every earlier column's update applied)
 *   u       float[cols, cols]; only the upper triangle j <= c is read; U_jj > 0
 *   scale, zero  float[rows, cols / group]: the grid of row r, column j is scale[r, j / group],
 *           zero[r, j / group]; group >= 1 divides cols
 *   qmin, qmax   integer code range, qmin < qmax, qmax - qmin <= 255, |qmin|, |qmax| <= 32767
 *   q_hat   float[rows, cols] written: (q - z) * s
 *   codes   uint8[rows, cols] written: q - qmin (for the W4 formats the stored nibble: qmin = -8
 *           symmetric, qmin = 0 asymmetric)
 *   err     float[rows, cols] written: column j's e = (w_j - q_hat_j) / U_jj
 *   rows, cols   1 <= rows < 2^31, 1 <= cols < 2^22
 * Column j, per row: q = rint(clamp(w_j / s + z, qmin, qmax)) (w_j / s taken as 0 when s == 0),
 * q_hat = (q - z) s, e = (w_j - q_hat) / U_jj, then w_c -= e U_jc for the block's columns c > j.
 * Every operation is fp32, rounded on its own in that order (products rounded before the
 * subtraction; no fused multiply-add; divisions correctly rounded).  The outputs must not overlap
 * each other or the inputs.  Asynchronous on `stream`; no allocation. */

/* One lazy block: columns [col0, col0 + bcols), 1 <= bcols <= 128, col0 + bcols <= cols.  Rows
 * run in parallel (a 16-lane team per row), the block's columns in sequence. */
int w4_gptq_block_update(float* w, const float* u, const float* scale, const float* zero,
                         int64_t rows, int64_t cols, int64_t group, int qmin, int qmax,
                         int64_t col0, int64_t bcols, float* q_hat, uint8_t* codes, float* err,
                         void* stream);

/* The lazy update after block [col0, col0 + bcols): W[:, i2:] -= E[:, col0:i2] U[col0:i2, i2:],
 * i2 = col0 + bcols, each element's sum over the block's columns taken in column order (products
 * rounded, then added), then subtracted.  Reads err's block columns; a no-op when i2 == cols. */
int w4_gptq_lazy_update(float* w, const float* u, const float* err, int64_t rows, int64_t cols,
                        int64_t col0, int64_t bcols, void* stream);

/* The whole column loop: for each block of `block` columns (1..128; the last one may be
 * narrower), w4_gptq_block_update then w4_gptq_lazy_update.  For layers of 2^23 weights and more,
 * after each block only the next block's columns are updated on `stream` and the columns beyond
 * on a helper stream of the library, joined back into `stream` before the next narrow update and
 * at the end (same results, bit for bit).  The helper stream and two events are created once per
 * device on the first such call made outside stream capture (no device memory is allocated);
 * until then, and for smaller layers, everything runs on `stream`.  Calls from several host
 * threads are serialized while they enqueue. */
int w4_gptq_quantize(float* w, const float* u, const float* scale, const float* zero, int64_t rows,
                     int64_t cols, int64_t group, int qmin, int qmax, int64_t block, float* q_hat,
                     uint8_t* codes, float* err, void* stream);

/* ------------------------------------------------------------------ 2:4 sparse GEMV -------- */

/* 2:4 structured sparsity (Do Quantization and Sparsity make LLM Inference Faster?, "Library 2:4
 * sparsity", "Custom CUDA 2:4 GEMV"): of every group of four weights along K two 16-bit values
 * are kept, with a 4-bit code per group holding their positions (i0 | i1 << 2, i0 < i1); stored
 * bytes are 56.25% of dense fp16.  Layout per row: values uint16[K/2] (the kept pair of group g at
 * 2g, 2g + 1), codes uint8[K/8] (group g in byte g/2, even groups in the low nibble).  The values
 * have the activations' 16-bit type. */
typedef enum { W4_S24_F16 = 0, W4_S24_BF16 = 1 } w4_s24_type_t;

/* w4_sparse24_compress: keep the two largest magnitudes of every group of four (the lower
 * position on equal magnitudes), rounded to nearest even to `xtype`.
 *   w       device float[N, K], read only; 16-byte aligned
 *   N, K    N >= 1; K a positive multiple of 32, K <= 16384
 *   values  device uint16[N, K/2], written; 16-byte aligned
 *   meta    device uint8[N, K/8], written; 4-byte aligned
 * Synchronizes `stream`.  Returns W4_ERR_NONFINITE if any weight is NaN or Inf. */
int w4_sparse24_compress(const float* w, int64_t N, int64_t K, int xtype, uint16_t* values,
                         uint8_t* meta, void* stream);

/* w4_sparse24_gemv: y[b, n] = sum over groups of v0 x[b, 4g + i0] + v1 x[b, 4g + i1], fp32
 * accumulation and output; the removed weights are never rebuilt.
 *   x       device [B, K] activations of `xtype` (bits), 16-byte aligned
 *   values, meta  as written by w4_sparse24_compress (alignment as there)
 *   N, K    as there; 1 <= B <= 8 (a lane multiplies each weight group with up to 8, 4, 2 or 1
 *           activation rows as its registers allow for the row length; larger batches stream the
 *           weights once per such slice)
 *   y       device float[B, N], written, 4-byte aligned; must not overlap an input
 * Asynchronous on `stream`; no allocation. */
int w4_sparse24_gemv(const uint16_t* x, const uint16_t* values, const uint8_t* meta, int xtype,
                     int64_t N, int64_t K, int64_t B, float* y, void* stream);

/* w4_sparse24_gemv_grouped: G 2:4 matrices that read the same activations (a layer's q, k and v,
 * or gate and up) in one launch, their row blocks one after another: y_g = x . W_g^T, each y_g
 * bitwise what w4_sparse24_gemv gives on member g alone (the same per-row arithmetic and launch
 * shape).  Fewer, fuller launches, as for w4_gemv_grouped.
 *   x         device [B, K] of `xtype`, shared; 16-byte aligned
 *   groups    G, 1 <= G <= W4_MAX_GROUP
 *   values, meta, y   host arrays of G device pointers (member g: [N_g, K/2], [N_g, K/8],
 *             float[B, N_g]; alignment as for w4_sparse24_gemv); no y_g may overlap another y_h or
 *             any input
 *   N         host array of G row counts, N_g >= 1, sum < 2^31
 *   xtype, K, B   as for w4_sparse24_gemv, shared
 * The host arrays are read during the call only.  Asynchronous on `stream`; no allocation. */
int w4_sparse24_gemv_grouped(const uint16_t* x, int groups, const uint16_t* const* values,
                             const uint8_t* const* meta, const int64_t* N, int xtype, int64_t K,
                             int64_t B, float* const* y, void* stream);

/* ------------------------------------------------------------------ measurement probes ------ */

/* Streaming-read ceiling probe: reads `bytes` (multiple of 16) from device `src` with 128-bit
 * loads, folds them, and writes one uint32 per workgroup to device `sink` (>= 4096 entries).
 * Used to measure the achievable HBM read bandwidth next to the GEMV (My Triton Kernel Ties
 * bitsandbytes, "The roofline first": measured, not spec-sheet, bandwidth).  Asynchronous. */
int w4_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Copy probe: dst[0:bytes] = src[0:bytes] with 128-bit loads and stores; bytes % 16 == 0;
 * the ranges must not overlap.  Asynchronous. */
int w4_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
