// Internal interface between the host entry points (attn_api.cpp) and the
// kernel launchers (*.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace eta {

// Tile shapes.  Forward: one workgroup per 128-query tile, streaming 64-key
// tiles.  Backward: one workgroup per 128-key tile, streaming 64-query tiles.
constexpr int kFwdBq = 128;
constexpr int kFwdBk = 64;
constexpr int kBwdBq = 64;
constexpr int kBwdBk = 128;
// dK / dV kernel at two waves per SIMD (bf16, no dropout, none / causal
// mask): 256-key tiles.
constexpr int kBwdKv2Bk = 256;
// Backward dQ (query-tile outer): the forward's tiling.
constexpr int kDqBq = 128;
constexpr int kDqBk = 32;
// Pipelined dQ kernel (bf16, (d, v) = (128, 128), (64, 128) or (64, 64)): 256-query tiles, 64-key
// tiles; with a bitmask at most kDqPipeMaxTk key tiles per row.
constexpr int kDqPipeBq = 256;
constexpr int kDqPipeBk = 64;
constexpr int kDqPipeMaxTk = 4096;
// Per-(batch, head) row padding of the backward's D and L2 arrays (a
// multiple of every query tile), so that whole tiles can be copied.
constexpr int kRowPad = 128;

// Dropout on the attention weights (p8 / 256 = drop probability; p8 = 0:
// none): counter-based keep decisions of kern_common.h, kept weights scaled
// by keep_inv = 256 / (256 - p8).
struct DropParams {
  uint32_t seed_lo, seed_hi;
  uint32_t p8;
  float keep_inv;
};

struct FwdParams {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  const uint8_t* map;  // bitmask tile map [mask units][tq][tk], else null
  const uint32_t* mask;
  int64_t mask_sb, mask_sh, mask_si;
  int64_t sq[3], sk[3], sv[3], so[3];
  int64_t n;         // query rows
  int64_t nk;        // key rows
  int64_t coff;      // causal: key j allowed for query i iff j <= i + coff
  int32_t B, H;
  int32_t tq, tk;
  int64_t total;     // B * H * tq work items
  int64_t grid_pad;  // total rounded up to a multiple of 8
  float scale2;      // c * log2(e): scores kept in the base-2 domain
  DropParams drop;
  // Split key ranges (pipelined bf16 forward only): splits > 1 runs
  // B H tq splits workgroups, split s taking its share of a query tile's key
  // tiles and writing its own normalised output and L (fp32) to Opart
  // [splits][B H][n][v] and Lpart [splits][B H][n]; fwd_merge_kernel then
  // combines them (ln-sum-exp of the L_s, exp(L_s - L) weights).
  int32_t splits;
  float* Opart;
  float* Lpart;
  // Debug tile counter (attn_debug_count_tiles), else null: each workgroup
  // adds the number of (query tile, key tile) pairs it computed.
  unsigned long long* tile_count;
};

struct BwdParams {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* L;
  float* Dn;     // -D_i = -<dO_i, O_i> (times P(keep) with dropout), fp32 [B, H, n_pad]
  float* L2;     // L_i log2(e) (+inf where L_i = -inf), fp32 [B, H, n_pad]
  // -L2_i / scale2 (scale2 = c log2(e), or 1e-30 for c = 0), fp32 [B, H,
  // n_pad], for the two-waves-per-SIMD dK / dV kernel (its score products
  // start from it); null otherwise.
  float* Ls;
  int64_t n_pad;  // row stride of Dn and L2: n rounded up to kRowPad; rows >= n hold 0 and L2 = +inf
  float* dQacc;  // fp32 [B, H, n, d] accumulator (unscaled by c)
  void* dQ;
  void* dK;
  void* dV;
  const uint8_t* map;
  const uint32_t* mask;
  int64_t mask_sb, mask_sh, mask_si;
  int64_t sq[3], sk[3], sv[3], so[3];
  int64_t n;     // query rows
  int64_t nk;    // key rows
  int64_t coff;  // causal offset, as in FwdParams
  int32_t B, H;
  int32_t tq, tk;  // key-tile-outer tiling: tq query tiles, tk key tiles of kBwdBk
  int64_t total;
  int64_t grid_pad;
  float scale;   // c
  float scale2;  // c * log2(e)
  // Query-tile-outer dQ kernel (deterministic path): tiles of kDqBq queries.
  const uint8_t* map_dq;  // bitmask tile map at the dQ tiling, else null
  int32_t tq_dq;
  int64_t total_dq;      // B H tq_dq dq_splits workgroups
  int64_t grid_pad_dq;
  // Key-range splits of the pipelined dQ kernel (1 = none): split s writes its
  // fp32 partial dQ (unscaled) for [B, H, n, d] to dQpart + s B H n d, and
  // bwd_dq_merge_kernel adds the splits in order and applies c.
  int32_t dq_splits;
  float* dQpart;
  DropParams drop;
  // Debug tile counters (attn_debug_count_tiles), else null: the key-tile-
  // outer kernel adds its computed tiles to tile_count_kv, the query-tile-
  // outer dQ kernel to tile_count_dq.
  unsigned long long* tile_count_kv;
  unsigned long long* tile_count_dq;
};

struct MapParams {
  const uint32_t* mask;
  int64_t mask_sb, mask_sh, mask_si;
  uint8_t* map;
  int64_t n, nk;  // query and key rows
  int64_t coff;   // causal offset
  int32_t B, H;
  int32_t units;  // distinct masks: H (batch-shared) or B * H
  int32_t bq, bk, tq, tk;
  int32_t mask_mode;
};

// Launchers return a hipError_t value as int (0 = success).
int launch_fwd(const FwdParams& p, int bf16, int d, int v, int mask_mode, void* stream);
// Key-range splits the forward uses for this problem (1 = none; > 1 only
// with the pipelined bf16 kernel, for few query tiles against many key tiles;
// with dropout too, since every split replays its keys' decisions).
inline int fwd_splits(int bf16, int64_t d, int64_t v, int64_t units, int64_t tq, int64_t tk) {
  if (!bf16 || !((d == 64 || d == 128) && (v == 64 || v == 128))) return 1;
  const int64_t wgs = units * tq;
  if (wgs >= 256) return 1;
  int64_t s = (512 + wgs - 1) / wgs;
  if (s > tk / 4) s = tk / 4;  // at least four key tiles per split
  if (s > 16) s = 16;
  return s < 2 ? 1 : (int)s;
}
int launch_fwd_merge(const FwdParams& p, int bf16, int v, void* stream);
int launch_bwd(const BwdParams& p, int bf16, int d, int v, int mask_mode, bool fused, void* stream);
int launch_bwd_dq(const BwdParams& p, int bf16, int d, int v, int mask_mode, void* stream);
// Pipelined dK / dV kernel of the deterministic path (bf16, d and v in {64, 128}).
bool bwd_kv_supported(int bf16, int d, int v, int mask_mode, int64_t tq);
int launch_bwd_kv(const BwdParams& p, int d, int v, int mask_mode, void* stream);
// The two-waves-per-SIMD dK / dV kernel of the deterministic path: bf16,
// (d, v) in {(128, 128), (64, 128), (64, 64)}, no dropout, none or causal
// mask.  The key-tile-outer tiling (and its bitmask map) follows this choice.
inline bool bwd_kv2_supported(int bf16, int64_t d, int64_t v, int mask_mode, bool fused, uint32_t drop_p8) {
  if (!bf16 || fused || drop_p8 != 0 || mask_mode == 2) return false;
  return (d == 128 && v == 128) || (d == 64 && v == 128) || (d == 64 && v == 64);
}
int launch_bwd_kv2(const BwdParams& p, int d, int v, int mask_mode, void* stream);
// Pipelined dQ kernel of the deterministic path; the tiling of the dQ pass
// (and of its bitmask tile map) follows this choice.
inline bool bwd_dq_pipe_supported(int bf16, int64_t d, int64_t v, int mask_mode, int64_t nk) {
  if (!bf16 || !((d == 128 && v == 128) || (d == 64 && v == 128) || (d == 64 && v == 64))) return false;
  return mask_mode != 2 || (nk + kDqPipeBk - 1) / kDqPipeBk <= kDqPipeMaxTk;
}
int launch_bwd_dq_pipe(const BwdParams& p, int d, int v, int mask_mode, void* stream);
// Key-range splits of the pipelined dQ kernel: > 1 only for few query tiles
// against many key tiles (B H tq_dq < 256), at least four key tiles each.
inline int dq_splits(int64_t units, int64_t tq_dq, int64_t tk_dq) {
  const int64_t wgs = units * tq_dq;
  if (wgs >= 256) return 1;
  int64_t s = (512 + wgs - 1) / wgs;
  if (s > tk_dq / 4) s = tk_dq / 4;
  if (s > 16) s = 16;
  return s < 2 ? 1 : (int)s;
}
int launch_bwd_dq_merge(const BwdParams& p, int d, void* stream);
// Keep decisions of dropout for rows [i0, i0 + rows) x keys [j0, j0 + cols)
// of one unit, as bytes 0 / 1 (row-major, `cols` per row); i0, j0 multiples of 4.
int launch_dropout_mask(const DropParams& d, uint32_t unit, int64_t i0, int64_t j0, int rows, int cols,
                        uint8_t* out, void* stream);
int launch_tile_map(const MapParams& p, void* stream);
int launch_bwd_pre(const BwdParams& p, int bf16, int d, int v, bool clear_dq, void* stream);
int launch_bwd_post(const BwdParams& p, int bf16, int d, void* stream);
const char* hip_error_string(int err);
int hip_last_launch_error();

// Opt-in launch timing (attn_timing_*): bracket one launch of kernel class
// `kind` with events on `stream`.  No-ops while timing is disabled.
void timing_begin(int kind, void* stream);
void timing_end(int kind, void* stream);
int timing_enable(int on);
int timing_read(double* ms, int64_t* launches);
void timing_reset();

// Static scratch of attn_bwd_noalloc (attn_scratch.hip): its size, and the
// device address of the current GPU's copy (resolved once per device with
// hipGetSymbolAddress; returns a hipError_t value, 0 = success).
size_t scratch_capacity();
int scratch_address(void** out);

// True when the (d, v) pair has compiled kernels.
inline bool supported_dims(int64_t d, int64_t v) {
  return (d == 64 && v == 64) || (d == 80 && v == 80) || (d == 128 && v == 128) ||
         (d == 64 && v == 128);
}

}  // namespace eta
