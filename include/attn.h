/*
 * attn.h -- C ABI of the MI355X (gfx950) exact tiled attention library.
 *
 * The operation (alphabetamath page, "Exact tiled softmax attention with
 * block-recomputed vector-Jacobian products", Inputs): for every (batch,
 * head) unit, positive n, d, v; Q, K in R^{n x d}; V in R^{n x v}; a real
 * scale c; nonempty allowed-key sets A_1..A_n.  With s_ij = c <Q_i, K_j>:
 * (Rectangular problems, with n query rows and nk key rows and a causal
 * offset, are described at attn_problem.nk.)
 *
 *   forward   O_i = sum_{j in A_i} exp(s_ij - L_i) V_j,
 *             L_i = ln sum_{j in A_i} exp(s_ij)            (natural log, fp32)
 *             (online softmax over key tiles, ob1 page part 1; maitreyasuin
 *             post, the tiled forward returning O and L = m + log l)
 *   backward  given dO (the upstream G), with D_i = <dO_i, O_i>,
 *             p_ij = exp(s_ij - L_i), dS_ij = p_ij (<dO_i, V_j> - D_i):
 *             dQ = c dS K,  dK = c dS^T Q,  dV = P^T dO
 *             (alphabetamath page, reverse procedure; ob1 page part 2;
 *             HarshvardhanJ/FlashAttention README, backward section)
 *
 * No n x n score or probability matrix is stored: every kernel rebuilds
 * score tiles on chip.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers.  The caller owns every buffer
 *   (inputs, outputs, mask, workspace); the library allocates nothing and
 *   keeps no state between calls except its loaded code objects.
 * - Q, K, V, O, dO, dQ, dK, dV are [B, H, n, .] (K, V, dK, dV: [B, H, nk, .]) with element strides
 *   (batch, head, row) given in attn_problem and a unit stride on the last
 *   dimension.  dQ, dK, dV use the strides of Q, K, V; dO uses those of O.
 *   Pointers must be 16-byte aligned and row/head/batch strides multiples
 *   of 16 bytes.  L (and the backward's internal D) are contiguous fp32
 *   [B, H, n].
 * - The kernels address one (batch, head) slice with 32-bit byte offsets,
 *   which sets three limits (ATTN_ERR_UNSUPPORTED beyond them): in every
 *   tensor, row 0 to the end of row n - 1 spans at most 2^31 - 1 bytes;
 *   n rounded up to 256 rows times the row stride stays below 2^32 bytes
 *   (tiles address the padding rows past the last one); and with
 *   deterministic = 0, one head's fp32 dQ accumulator, n d 4 bytes, is at
 *   most 2^31 - 1 bytes.  Batch and head offsets are 64-bit.
 * - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *   asynchronously on it; nothing synchronises.
 * - Every argument is validated before anything is launched; on an error
 *   status nothing has been written.  attn_last_error() then returns a
 *   thread-local message describing the failure.
 * - Q, K, V may alias each other (self-attention).  Outputs must not
 *   overlap any input or each other (ATTN_ERR_ALIAS).
 * - Empty allowed rows are outside the contract (A_i must be nonempty);
 *   the library still defines them: O_i = 0, L_i = -inf, and such rows
 *   contribute nothing to dQ, dK, dV.
 */
#ifndef EXACT_TILED_ATTN_H
#define EXACT_TILED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* B, H, n, d or v < 1, or a size overflows */
  ATTN_ERR_STRIDE = 3,      /* misaligned pointer or stride, or overlapping rows */
  ATTN_ERR_DTYPE = 4,       /* unknown element type */
  ATTN_ERR_MASK = 5,        /* unknown mask mode, or bitmask mode without mask */
  ATTN_ERR_UNSUPPORTED = 6, /* (d, v) pair or option not compiled in, or past a size limit */
  ATTN_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than attn_workspace_size */
  ATTN_ERR_ALIAS = 8,       /* an output overlaps an input or another output */
  ATTN_ERR_HIP = 9          /* a HIP launch error (message in attn_last_error) */
} attn_status;

typedef enum {
  ATTN_F32 = 0,  /* fp32 inputs and outputs, fp32 MFMA, fp32 accumulation */
  ATTN_BF16 = 1  /* bf16 inputs and outputs, bf16 MFMA, fp32 accumulation */
} attn_dtype;

/* The allowed-key sets A_i (alphabetamath page, Inputs: membership read on
 * demand; a caller-owned mask representation is input storage). */
typedef enum {
  ATTN_MASK_NONE = 0,    /* A_i = {0..n-1} */
  ATTN_MASK_CAUSAL = 1,  /* A_i = {j <= i + causal_offset} (ob1 page, part 3: block causal) */
  ATTN_MASK_BITMASK = 2  /* explicit: bit (j & 31) of word j >> 5 of row i */
} attn_mask_mode;

typedef struct {
  int64_t B, H;           /* batch and head counts */
  int64_t n;              /* sequence length (queries = keys) */
  int64_t d, v;           /* key/query dim and value dim; (d, v) in
                             {(64,64), (80,80), (128,128), (64,128)} */
  int32_t dtype;          /* attn_dtype */
  int32_t mask_mode;      /* attn_mask_mode */
  double scale;           /* c: any finite real, including 0 and negative */
  const uint32_t* mask;   /* BITMASK only: device words, LSB first, pad bits ignored */
  int64_t mask_sb;        /* mask strides in uint32 words: batch (0 = shared), */
  int64_t mask_sh;        /*   head, */
  int64_t mask_si;        /*   row (>= ceil(nk/32)) */
  int64_t sq[3];          /* element strides [batch, head, row] of Q and dQ */
  int64_t sk[3];          /* ... of K and dK */
  int64_t sv[3];          /* ... of V and dV */
  int64_t so[3];          /* ... of O and dO */
  int32_t deterministic;  /* bwd: 0 = dQ by fp32 atomics in the key-tile-outer
                             kernel; 1 = dQ by a separate query-tile-outer
                             kernel (bitwise reproducible, no atomics, and
                             the faster choice on MI355X: its fp32 atomic
                             adds run at about 1.3 TB/s, so with 0 the
                             backward takes about twice as long) */
  int32_t reserved;       /* must be 0 */
  /* Rectangular problems (maitreyasuin page, the tiled forward: Tq query
   * rows against Tk key rows).  nk: rows of K, V, dK, dV; 0 means nk = n.
   * causal_offset (CAUSAL only, else it must be 0): key j is allowed for
   * query i iff j <= i + causal_offset.  0 is the square causal mask;
   * nk - n aligns the last query with the last key (queries appended after
   * a cache of keys); a shard of queries starting at absolute position qp
   * against keys starting at kp uses qp - kp.  |causal_offset| <= 2^30.
   * Rows left with no allowed key get O_i = 0, L_i = -inf (see above), so
   * that results over disjoint key ranges merge exactly:
   * L = ln sum_s exp(L_s), O = sum_s exp(L_s - L) O_s. */
  int64_t nk;
  int64_t causal_offset;
  /* Dropout on the attention weights (the alphabetamath page names dropout
   * only as an extension whose reverse pass must replay the forward's
   * realised mask).  dropout_p in [0, 1) is used in units of 1/256:
   * p8 = round(256 dropout_p); p8 = 0 disables dropout.  Pair (i, j) of
   * unit u = b H + h is kept iff its 8-bit draw is >= p8: byte j % 4 of word
   * i % 4 of Philox4x32-10 (Salmon et al., SC 2011) at counter
   * (j / 4, i / 4, u, 0) and key (dropout_seed mod 2^32, dropout_seed div
   * 2^32).  O_i = sum_j P_ij Z_ij V_j * 256 / (256 - p8), with P the
   * undropped softmax, whose L is returned; attn_bwd with the same seed and
   * dropout_p regenerates Z.  Every forward and backward kernel draws Z
   * itself, the pipelined bf16 ones included, so dropout changes neither
   * the kernels chosen nor the key-range splits. */
  double dropout_p;
  uint64_t dropout_seed;
} attn_problem;

/* Bytes of device workspace attn_fwd (is_bwd = 0) or attn_bwd (is_bwd = 1)
 * needs for this problem.  Forward: the tile map of bitmask mode, and, when
 * few query tiles face many key tiles (bf16, d and v in {64, 128}, no
 * dropout), the partial results of the key-range splits, S B H n (v + 1) * 4
 * bytes for S <= 16 splits (0 bytes if neither applies).  Backward: D and
 * L log2(e) (4 B H n_pad bytes each, n_pad = n rounded up to 128), plus
 * -L log2(e) / (c log2(e)) alike when deterministic = 1 with bf16, (d, v) in
 * {(128,128), (64,128), (64,64)}, no dropout and a none or causal mask (the
 * two-waves-per-SIMD dK / dV kernel starts its score products from it), plus the
 * fp32 dQ accumulator (4 B H n d bytes) when deterministic = 0, plus the
 * bitmask tile map(s), plus, when deterministic = 1 and few query tiles face
 * many key tiles (bf16 with (d, v) in {(128,128), (64,128), (64,64)}), the
 * dQ kernel's key-range partials, S B H n d * 4 bytes for
 * S <= 16 splits; every region 256-byte aligned.  Validates the problem like
 * the compute calls. */
attn_status attn_workspace_size(const attn_problem* p, int is_bwd, size_t* bytes);

/* Forward: O [B,H,n,v] (dtype) and L [B,H,n] (fp32, natural-log logsumexp
 * of the scaled allowed scores).  Kernels: bitmask tile classification
 * (bitmask mode only), then one fused tiled kernel per call; with key-range
 * splits (see attn_workspace_size) each split writes its own output and L,
 * which a merge kernel combines exactly (L = ln sum_s e^{L_s},
 * O = sum_s e^{L_s - L} O_s).  Rectangular
 * problems: O and L have n rows, K and V nk rows. */
attn_status attn_fwd(const attn_problem* p, const void* Q, const void* K, const void* V,
                     void* O, float* L, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Backward: dQ, dK, dV (dtype) from Q, K, V, the forward's O and L, and the
 * upstream gradient dO.  Kernels: D = rowsum(dO o O) (clearing the dQ
 * accumulator when deterministic = 0), bitmask tile classification (bitmask
 * mode), the key-tile-outer recompute kernel (dK, dV in registers), then
 * either dQ by fp32 atomics in that kernel plus a conversion pass
 * (deterministic = 0; dQ may differ run to run in the last bits) or a
 * query-tile-outer dQ kernel (deterministic = 1; bitwise reproducible).
 * With key-range splits of that kernel (see attn_workspace_size) each split
 * writes an fp32 partial dQ and a merge kernel adds them in split order
 * (still bitwise reproducible). */
attn_status attn_bwd(const attn_problem* p, const void* Q, const void* K, const void* V,
                     const void* O, const void* dO, const float* L,
                     void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Backward that allocates nothing: for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same operation, arguments, results and errors as
 * attn_bwd, without the workspace arguments: the workspace is a static
 * 64 MiB device array of the library, of which each GPU holds its own copy
 * from the first call on that GPU until the process ends.  Problems whose
 * attn_workspace_size (is_bwd = 1) exceeds 64 MiB are refused with
 * ATTN_ERR_WORKSPACE before anything runs (the atomic path's fp32 dQ
 * accumulator, 4 B H n d bytes, reaches that size first).  Every region the
 * kernels read is written earlier in the same call, so a call never sees an
 * earlier call's contents; but all calls on one GPU share the array, so
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and must be serialised by the caller. */
attn_status attn_bwd_noalloc(const attn_problem* p, const void* Q, const void* K, const void* V,
                             const void* O, const void* dO, const float* L,
                             void* dQ, void* dK, void* dV, void* stream);

/* Debug: the (query tile x key tile) classification the forward (is_bwd=0),
 * key-tile-outer backward (is_bwd=1) or query-tile-outer dQ (is_bwd=2)
 * kernels use, 0 = empty (skipped), 1 = partial
 * (masked inside), 2 = full (no masking), as uint8 [units, tq, tk] with
 * units = 1 for none/causal masks (shared by every head), else the number
 * of distinct masks (H if mask_sb == 0, else B*H, in (b, h) order).
 * Writes *bq, *bk (tile sizes) and *tq, *tk; if map_dev is NULL only the
 * sizes are returned, else map_bytes must hold units*tq*tk bytes.  The
 * workspace arguments are reserved (pass NULL, 0). */
attn_status attn_debug_tile_map(const attn_problem* p, int is_bwd, uint8_t* map_dev,
                                size_t map_bytes, int32_t* bq, int32_t* bk, int32_t* tq,
                                int32_t* tk, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Debug: the dropout keep decisions (1 = kept, 0 = dropped) the kernels use
 * for unit (b, h), query rows [i0, i0 + rows) and keys [j0, j0 + cols), as
 * rows * cols bytes, row-major, written to out_dev (out_bytes must hold
 * them).  i0 and j0 must be multiples of 4, rows and cols >= 1; the problem
 * must have dropout enabled (ATTN_ERR_UNSUPPORTED otherwise). */
attn_status attn_debug_dropout_mask(const attn_problem* p, int64_t b, int64_t h, int64_t i0, int64_t j0,
                                    int32_t rows, int32_t cols, uint8_t* out_dev, size_t out_bytes,
                                    void* stream);

/* Debug: count the tiles the kernels compute.  The classification of
 * attn_debug_tile_map fixes which (query tile x key tile) pairs hold an
 * allowed pair; the kernels must compute exactly those and skip the rest
 * (alphabetamath page, forward procedure: blocks whose intersection with A_i
 * is empty are skipped; ob1 page, part 3: key blocks right of the causal
 * diagonal are skipped).  While counters_dev is set, every forward kernel
 * adds the number of tiles it computed (at the forward's tiling, is_bwd = 0
 * of attn_debug_tile_map) to counters_dev[0], every key-tile-outer backward
 * kernel to counters_dev[1] (is_bwd = 1), every query-tile-outer dQ kernel
 * to counters_dev[2] (is_bwd = 2), with one 64-bit atomic add per
 * workgroup; key-range splits add their shares.  counters_dev: three
 * caller-owned uint64 device words, 8-byte aligned, cleared by the caller;
 * NULL (the default) switches counting off.  A process-wide setting, not
 * thread-safe; ATTN_ERR_STRIDE for a misaligned pointer. */
attn_status attn_debug_count_tiles(uint64_t* counters_dev);

/* Kernel classes reported by the timing facility below. */
typedef enum {
  ATTN_KERNEL_TILE_MAP = 0, /* bitmask tile classification */
  ATTN_KERNEL_FWD = 1,      /* forward */
  ATTN_KERNEL_BWD_PRE = 2,  /* D = rowsum(dO o O), accumulator clearing */
  ATTN_KERNEL_BWD = 3,      /* key-tile-outer backward */
  ATTN_KERNEL_BWD_POST = 4, /* dQ conversion (deterministic = 0) */
  ATTN_KERNEL_BWD_DQ = 5,   /* query-tile-outer dQ (deterministic = 1) */
  ATTN_KERNEL_FWD_MERGE = 6, /* merge of the forward's key-range splits */
  ATTN_KERNEL_BWD_DQ_MERGE = 7, /* sum of the dQ kernel's key-range splits */
  ATTN_KERNEL_COUNT = 8
} attn_kernel;

/* Opt-in kernel timing (off by default; not thread-safe; for measurement
 * tools).  While enabled, every kernel the library launches is bracketed by
 * two HIP events recorded on the launch stream.  attn_timing_read waits for
 * the recorded events, adds each launch's duration to ms[kind] and counts it
 * in launches[kind] (both arrays of ATTN_KERNEL_COUNT entries, accumulated
 * since the last read or reset), then recycles the events.  Disabling or
 * resetting discards pending measurements. */
attn_status attn_timing_enable(int on);
attn_status attn_timing_read(double* ms, int64_t* launches);
attn_status attn_timing_reset(void);

/* Static description of a status code. */
const char* attn_status_str(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* attn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch (0.5.0 added
 * attn_debug_count_tiles, 0.6.0 attn_bwd_noalloc). */
int32_t attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_ATTN_H */
