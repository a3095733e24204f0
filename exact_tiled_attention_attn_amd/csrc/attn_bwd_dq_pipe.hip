// Backward, query-tile-outer dQ kernel for bf16 with (d, v) = (128, 128), (64, 128) or (64, 64): the
// second kernel of the deterministic backward (dK and dV come from the
// key-tile-outer kernel).
//
// Method (alphabetamath page, reverse procedure; ob1 page, part 2;
// HarshvardhanJ README, backward section): with the forward's L and
// D_i = <dO_i, O_i>, for every allowed (i, j) recompute s_ij = c <Q_i, K_j>,
// p_ij = exp(s_ij - L_i), dS_ij = p_ij (<dO_i, V_j> - D_i) and accumulate
// dQ_i += c dS_ij K_j.  Each workgroup owns 256 query rows and streams the
// key tiles in ascending order, so every dQ row is summed by one lane in a
// fixed order: the result is deterministic and needs no atomics.  Tiles with
// no allowed pair are skipped; only partially allowed tiles are masked (ob1
// page, part 3).
//
// gfx950 design.  One workgroup per CU; each of its 4 waves owns 64 queries
// as two halves of 32 (lane column = query) and keeps their Q and dO rows in
// AGPRs as MFMA B operands and their dQ^T accumulators in AGPRs, so L_i and
// D_i are per-lane constants; the score accumulators live in VGPRs, where
// the vector ALUs read them without copies (MFMAs written as inline
// assembly with explicit register classes).  Key tiles of 64 rows are processed as two
// chunks of 32 keys.  Per chunk, S^T = K Q^T and dP^T = V dO^T: every K or V
// row operand read from LDS feeds the MFMAs of both halves, and the dP^T
// accumulators start from -D_i, so that they come out as dP - D.  The vector
// ALUs form P = exp2(c log2(e) s - L_i log2(e)) and dS = P (dP - D) in the
// score registers, whose packed form is the B operand of dQ^T += K^T dS^T;
// its K^T operand comes from transposed reads of the same K tile.  The
// chunks form a software pipeline: the S / dP products of chunk k+1 run on
// the matrix cores while the vector ALUs work on chunk k, then chunk k's dQ
// products run; the instruction order is pinned with scheduling barriers.
// K, V (and the bitmask words) are copied from HBM straight into a 4-stage
// ring of LDS tiles (buffer_load ... lds, issued from inline assembly and
// counted with vmcnt) two tiles ahead of their use, with one barrier per
// tile; the copies of a tile are spread over the MFMAs of a chunk.  Tile rows
// are padded by 16 bytes and the key rows of each group of 16 are taken in
// transposed order (4 u + v -> u + 4 v) by the score products, so that the
// transposed K^T reads cover rows 4 apart: both kinds of read are then free
// of bank conflicts and every LDS read address is one per-lane register plus
// a constant.
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {

#ifndef ETA_DQ_PREFETCH_A
#define ETA_DQ_PREFETCH_A 3
#endif
#ifndef ETA_DQ_PREFETCH_B
#define ETA_DQ_PREFETCH_B 3
#endif
// LDS operand prefetch depth, in operands (each feeds two MFMAs), of the two phases.
constexpr int kDqPrefetchA = ETA_DQ_PREFETCH_A, kDqPrefetchB = ETA_DQ_PREFETCH_B;

// The score products use the explicit-register MFMAs of kern_common.h: their
// accumulators live in VGPRs (read directly by the vector ALUs) and their Q /
// dO operands in AGPRs; the dQ^T products accumulate in AGPRs.  Wait states
// the compiler cannot see are kept by construction: every score result is
// read at least one 16-MFMA phase after it is written (s_nop after the
// prologue's products), the packed dS operands are written two or more
// instructions before their first use (s_nop 1 at the start of the second
// phase), and accumulation chains use the same registers for the
// accumulator and the result.

template <int D, int DV>
struct DqPipeShape {
  static constexpr int NW = 4;
  static constexpr int BQ = kDqPipeBq;  // queries per workgroup: 64 per wave, two halves of 32
  static constexpr int BK = kDqPipeBk;  // keys per tile: two chunks of 32
  static constexpr int NSTAGE = 4;      // LDS ring: tiles j .. j+2 resident or in flight
  static constexpr int NQF = D / 16, NVF = DV / 16;  // Q / dO fragments per lane and half
  static constexpr int NDB = D / 32;                 // 32-row blocks of dQ^T
  static constexpr int NR = NQF + NVF;               // K / V row operands per chunk (2 MFMAs each)
  static constexpr int NB = 2 * NDB;                 // K^T operands per chunk (2 key steps; 2 MFMAs each)
  using KT = PadTile<D * 2, 16>;
  using VT = PadTile<DV * 2, 16>;
  static constexpr int KS = KT::kStride, VS = VT::kStride;
  static constexpr int KTILE = BK * KS, VTILE = BK * VS;
  static constexpr int KWINS = KTILE / 1024, VWINS = VTILE / 1024;  // 1 KB fill windows per tile
  // Copies per wave and tile (KWIN / VWIN): a contiguous run of windows, the
  // last of which is an empty copy for some waves.
  static constexpr int KWIN = (KWINS + NW - 1) / NW, VWIN = (VWINS + NW - 1) / NW;
  static constexpr int MWORDS = BK / 32;         // bitmask words per query row and tile
  static constexpr int MTILE = BQ * MWORDS * 4;  // bitmask bytes per stage
  static constexpr int MAXTK = 4096;             // bitmask: key tiles whose classes are staged in LDS
  static_assert(KTILE % 1024 == 0 && VTILE % 1024 == 0, "whole fill windows");
  static_assert(BQ == 256 && BK == 64, "64 queries per wave, two chunks of 32 keys");
  static_assert(MTILE == NW * 2 * 256, "two 256-byte mask-word copies per wave");
};

template <int D, int DV, int MASK, bool DROP>
__global__ __launch_bounds__(256, 1) void bwd_dq_pipe_kernel(BwdParams p) {
  using S = DqPipeShape<D, DV>;
  __shared__ __attribute__((aligned(1024))) char kts[S::NSTAGE * S::KTILE];
  __shared__ __attribute__((aligned(1024))) char vts[S::NSTAGE * S::VTILE];
  __shared__ __attribute__((aligned(16))) char mws[MASK == kMaskBitmask ? S::NSTAGE * S::MTILE : 16];
  __shared__ uint8_t cls_s[MASK == kMaskBitmask ? S::MAXTK : 1];
  __shared__ __attribute__((aligned(1024))) char spare[4096];  // target of the padding copies (any immediate offset)

  const int64_t logical0 = xcd_logical(blockIdx.x, p.grid_pad_dq, p.total_dq);
  if (logical0 < 0) return;
  const int split = (int)(logical0 % p.dq_splits);  // key-range split (0 when not splitting)
  const int64_t logical = logical0 / p.dq_splits;
  const int unit = (int)(logical / p.tq_dq);
  const int qt = p.tq_dq - 1 - (int)(logical % p.tq_dq);  // heaviest causal tiles first
  const int b = unit / p.H, h = unit % p.H;
  const int n = (int)p.n, nk = (int)p.nk, coff = (int)p.coff;  // query rows, key rows, causal offset
  const int q0 = qt * S::BQ;
  const int tk = (nk + S::BK - 1) / S::BK;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int g1 = (lane >> 4) & 1;
  const int qa = q0 + 64 * w + (lane & 31);  // query of half 0; half 1: qa + 32

  const int qrow = (int)p.sq[2] * 2, krow = (int)p.sk[2] * 2;
  const int vrow = (int)p.sv[2] * 2, orow = (int)p.so[2] * 2;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * 2;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * 2;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * 2;
  const char* dOb = (const char*)p.dO + ((int64_t)b * p.so[0] + (int64_t)h * p.so[1]) * 2;
  const uint32_t* mbase = nullptr;
  if constexpr (MASK == kMaskBitmask) mbase = p.mask + b * p.mask_sb + h * p.mask_sh;

  // Per-lane row statistics of the two halves: L log2(e) (+inf for rows past
  // n or with L = -inf, so that p = 0) and -D (with dropout -D P(keep)).
  float l2[2], dn[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = qa + 32 * u;
    l2[u] = q < n ? p.L2[(int64_t)unit * p.n_pad + q] : INFINITY;
    dn[u] = q < n ? p.Dn[(int64_t)unit * p.n_pad + q] : 0.f;
  }

  // Key-tile sequence: ascending, up to the last tile that can hold an
  // allowed pair (causal: the tile holding the last key the last row allows); bitmask
  // tiles come from the tile map, staged in LDS so that the loop issues no
  // loads of its own.
  int kt_end = tk;
  if constexpr (MASK == kMaskCausal) {
    const int k_hi = (q0 + S::BQ < n ? q0 + S::BQ : n) - 1 + coff;  // last key any row allows
    kt_end = k_hi < 0 ? 0 : (k_hi / S::BK + 1 < tk ? k_hi / S::BK + 1 : tk);
  }
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    const uint8_t* map_row = p.map_dq + (mu * p.tq_dq + qt) * (int64_t)tk;
    for (int t = tid; t < tk; t += 256) cls_s[t] = map_row[t];
  }
  auto tile_class = [&](int kt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return cls_s[kt];
    return classify_analytic(MASK, q0, S::BQ, (int64_t)kt * S::BK, S::BK, n, nk, coff);
  };
  // Partially allowed among the visited (nonempty) tiles, with 32-bit scalar
  // arithmetic: the first kt_full tiles are full (every key exists and, with
  // the causal mask, is allowed for the tile's first row), later ones partial.
  int kt_full = nk / S::BK;
  if constexpr (MASK == kMaskCausal) {
    const int r = q0 + coff - (S::BK - 1);  // last tile start a first-row-full tile can have
    const int f = r < 0 ? 0 : r / S::BK + 1;
    kt_full = f < kt_full ? f : kt_full;
  }
  auto tile_partial = [&](int kt) -> bool {
    if constexpr (MASK == kMaskBitmask) return cls_s[kt] == kTilePartial;
    return kt >= kt_full;
  };
  auto next_tile = [&](int kt) -> int {  // next (higher) tile with an allowed pair, or -1
    if (kt < 0) return -1;
    if constexpr (MASK != kMaskBitmask) return kt + 1 < kt_end ? kt + 1 : -1;
    for (int t = kt + 1; t < kt_end; ++t)
      if (tile_class(t) != kTileEmpty) return t;
    return -1;
  };

  // Q and dO rows of the wave's queries (B operands; lane column = query).
  bf16x8 qf[2][S::NQF], of[2][S::NVF];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb, (int64_t)n * qrow);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(dOb, (int64_t)n * orow);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int s = 0; s < S::NQF; ++s)
        qf[u][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, (qa + 32 * u) * qrow + (16 * s + 8 * hh) * 2, 0, 0));
#pragma unroll
      for (int s = 0; s < S::NVF; ++s)
        of[u][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, (qa + 32 * u) * orow + (16 * s + 8 * hh) * 2, 0, 0));
    }
  }
  f32x16 dq[2][S::NDB], dinit[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int i = 0; i < S::NDB; ++i) dq[u][i] = f32x16{};
#pragma unroll
    for (int r = 0; r < 16; ++r) dinit[u][r] = dn[u];
  }
  // Dropout (DROP): dS = P (Z dP / keep - D) = P (Z dP - keep D) / keep.  The
  // dP accumulators start from -keep D as they start from -D without
  // dropout, a dropped pair takes -keep D instead (one bit select), and the
  // 1 / keep joins c at the end.  The keep decisions Z of kern_common.h are
  // regenerated per 32-key chunk.  Per half u, lane (hh, quad position e) draws key block
  // 4 hh + e of the chunk for its quad's query block (counter (key / 4,
  // query / 4, unit, 0)); the call's 16 keep bits are packed as bit
  // 8 (key % 4) + 4 + query % 4.  Register r = 4 g + e' of a half holds key
  // 16 (g / 2) + 2 (g % 2) + hh + 4 e' of the chunk (the perm() order), i.e.
  // key block 4 (g / 2) + e', key 2 (g % 2) + hh in it: the call of the lane
  // in half g / 2 at quad position e', bit dsh + 16 (g % 2).  The next chunk's
  // calls are drawn during a step's second phase (where the vector ALUs are
  // idle) and shared by one half swap and quad broadcasts.
  const uint32_t dsh = 4u + (uint32_t)(lane & 3) + 8u * (uint32_t)hh;
  const KeepConsts kq = keep_consts(p.drop.p8);
  uint32_t dc[2][4] = {}, dm[2] = {0u, 0u}, dM[2][2][4] = {};
  auto draw_init = [&](int key0) {  // first key of the chunk (a multiple of 32)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      dc[u][0] = ((uint32_t)key0 >> 2) + 4u * (uint32_t)hh + (uint32_t)(lane & 3);
      dc[u][1] = (uint32_t)(qa + 32 * u) >> 2;
      dc[u][2] = (uint32_t)unit;
      dc[u][3] = 0u;
      dm[u] = 0u;
    }
  };
  auto draw_item = [&](int t) {  // call t / 14: rounds 0..9, then the keep bits of its four words
    const int u = t / 14, k = t % 14;
    if (k < 10) philox_round(dc[u][0], dc[u][1], dc[u][2], dc[u][3], p.drop.seed_lo, p.drop.seed_hi, k);
    else dm[u] = pack_keep(dm[u], keep_flags(dc[u][k - 10], kq), k - 10);
  };
  auto draw_share = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      auto sw = __builtin_amdgcn_permlane32_swap(dm[u], dm[u], false, false);  // [0]: half 0's call, [1]: half 1's
      dM[u][0][0] = quad_bcast<0>(sw[0]);
      dM[u][0][1] = quad_bcast<1>(sw[0]);
      dM[u][0][2] = quad_bcast<2>(sw[0]);
      dM[u][0][3] = quad_bcast<3>(sw[0]);
      dM[u][1][0] = quad_bcast<0>(sw[1]);
      dM[u][1][1] = quad_bcast<1>(sw[1]);
      dM[u][1][2] = quad_bcast<2>(sw[1]);
      dM[u][1][3] = quad_bcast<3>(sw[1]);
    }
  };
  auto keep_mask = [&](int u, int r) -> uint32_t {  // all ones iff register r of half u is kept
    const int g = r >> 2, e = r & 3;
    return (uint32_t)__builtin_amdgcn_sbfe((int)dM[u][g >> 1][e], dsh + 16u * (uint32_t)(g & 1), 1u);
  };

  // ---- tile fills ----------------------------------------------------------
  // Wave w copies a contiguous run of 1 KB windows of each tile: KB = KWINS /
  // NW of them, plus one more for the first KX = KWINS % NW waves (the others
  // issue that item as an empty copy into the spare window, so that every
  // wave issues the same instructions).  Consecutive windows share one M0
  // value in groups of four: the copy's immediate offset selects the window
  // and is taken off the per-lane source offsets.
  constexpr int KB = S::KWINS / S::NW, KX = S::KWINS % S::NW;
  constexpr int VB = S::VWINS / S::NW, VX = S::VWINS % S::NW;
  static_assert(S::KWIN == KB + (KX > 0) && S::VWIN == VB + (VX > 0), "window counts");
  const int kfirst = w * KB + (w < KX ? w : KX), vfirst = w * VB + (w < VX ? w : VX);
  int ksrc[S::KWIN], vsrc[S::VWIN];
#pragma unroll
  for (int i = 0; i < S::KWIN; ++i)
    ksrc[i] = (int)((uint32_t)S::KT::fill_src((kfirst + i) * 1024 + 16 * lane, krow) - (uint32_t)((i % 4) * 1024));
#pragma unroll
  for (int i = 0; i < S::VWIN; ++i)
    vsrc[i] = (int)((uint32_t)S::VT::fill_src((vfirst + i) * 1024 + 16 * lane, vrow) - (uint32_t)((i % 4) * 1024));
  // Key row of the tile behind lane m % 32 of a score product's A operand:
  // groups of 16 rows taken in transposed order, 4 u + v -> u + 4 v.
  auto perm = [](int l) { return (l & ~15) + ((l & 15) >> 2) + 4 * (l & 3); };
  const uint32_t ks_l = lds_address(kts), vs_l = lds_address(vts), ms_l = lds_address(mws);
  const uint32_t sp_l = lds_address(spare);
  // Per tile every wave issues KWIN + VWIN copies and, with a bitmask, two
  // more (mask words of 32 query rows each).
  constexpr int kBm = MASK == kMaskBitmask;
  constexpr int kF = S::KWIN + S::VWIN + 2 * kBm;
  const i32x4 r_none = rsrc_words(Kb, 0);
  // Mask words: copy i of wave w covers query rows 64 w + 32 i + lane / 2 of
  // the tile, word lane % 2 of the key tile; row r lands at bytes 8 r.
  auto fill_mask = [&](const i32x4& rm, int st, int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * w + 32 * i + lane / 2;
      fill4(rm, ms_l + st * S::MTILE + (64 * w + 32 * i) * 8,
            (int)(((int64_t)r * p.mask_si + (k0 >> 5) + (lane & 1)) * 4));
    }
  };
  auto mask_rsrc = [&](int64_t rows) { return rsrc_words(mbase + (int64_t)q0 * p.mask_si, rows * p.mask_si * 4); };
  // Item i of this wave's run over a tile at LDS byte address `tile`.
  auto win_item = [&](const i32x4& r, uint32_t tile, int first, int nb, int nx, const auto& src, int i) {
    const bool extra = i == nb;
    const bool real = !extra || w < nx;
    if (i % 4 == 0 || extra)  // group start, or the item that may be an empty copy
      set_m0(real ? tile + (first + 4 * (i / 4)) * 1024 : sp_l);  // an empty copy lands at sp_l + (i % 4) KB
    // An empty copy keeps the resource's address and takes an empty range.
    fill16_off(i32x4{r[0], r[1], real ? r[2] : 0, r[3]}, src[i], i % 4);
  };
  auto kwin = [&](const i32x4& rk, int st, int i) { win_item(rk, ks_l + st * S::KTILE, kfirst, KB, KX, ksrc, i); };
  auto vwin = [&](const i32x4& rv, int st, int i) { win_item(rv, vs_l + st * S::VTILE, vfirst, VB, VX, vsrc, i); };
  auto fill = [&](int kt, int st) {  // kt < 0: empty ranges, same instructions
    const int k0 = kt < 0 ? 0 : kt * S::BK;
    const int64_t rows = kt < 0 ? 0 : nk - k0;
    const i32x4 rk = rsrc_words(Kb + (int64_t)k0 * krow, rows * krow);
    const i32x4 rv = rsrc_words(Vb + (int64_t)k0 * vrow, rows * vrow);
#pragma unroll
    for (int i = 0; i < S::KWIN; ++i) kwin(rk, st, i);
#pragma unroll
    for (int i = 0; i < S::VWIN; ++i) vwin(rv, st, i);
    if constexpr (MASK == kMaskBitmask) fill_mask(mask_rsrc(kt < 0 ? 0 : n - q0), st, k0);
  };
  // The same copies split in two, for the fill issued inside a pipeline step:
  // the first FK + FV items (issued one per four MFMAs of the step's first
  // phase) and the rest (the extra items, mask words), issued first.  kt < 0
  // copies nothing (empty buffer ranges) but issues the same instructions.
  constexpr int FK = KB, FV = VB;
  static_assert(4 * (FK + FV) <= 2 * S::NR, "one spread copy per four first-phase MFMAs at most");
  i32x4 frk, frv;
  int fst = 0;
  // Buffer resource of the rows of key tile kt of a [nk, row] slice with rb
  // bytes per row; the host bounds (nk - 1) rb + the row width by 2^31 - 1,
  // so the products fit in 32 bits.  kt < 0: an empty range.
  auto tile_words = [&](const void* base, int kt, int rb) -> i32x4 {
    const uint32_t k0 = kt < 0 ? 0u : (uint32_t)(kt * S::BK);
    const uint32_t nb = kt < 0 ? 0u : (uint32_t)(nk - (int)k0) * (uint32_t)rb;
    const uint64_t a = reinterpret_cast<uint64_t>(base) + k0 * (uint32_t)rb;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)(nb < 0x7FFFFFFFu ? nb : 0x7FFFFFFFu), 0x00020000};
  };
  // The next in-step fill, planned in chunk 0's second phase (its scalar work
  // issues under the MFMAs): K / V resources, key tile and target stage.
  int fkt = -1;
  // Without a bitmask the visited key tiles are consecutive (ascending): the
  // next fill's resources follow from the previous ones by one tile's bytes.
  // ak / av are the byte addresses of the planned tile's K and V rows, nkb /
  // nvb the bytes from there to row nk, unclamped (they wrap once past the
  // last tile, whose fills then take empty ranges, so neither value is used
  // there; the resources take them clamped below 2^31).
  uint64_t ak = 0, av = 0;
  uint32_t nkb = 0, nvb = 0;
  const uint32_t ck = (uint32_t)(S::BK * krow), cv = (uint32_t)(S::BK * vrow);
  auto plan_start = [&](int kt) {  // state of tile kt (kt < 0 only ever precedes empty fills)
    const int t = kt < 0 ? 0 : kt;
    ak = reinterpret_cast<uint64_t>(Kb) + (uint64_t)((uint32_t)t * ck);
    av = reinterpret_cast<uint64_t>(Vb) + (uint64_t)((uint32_t)t * cv);
    nkb = (uint32_t)(nk - t * S::BK) * (uint32_t)krow;
    nvb = (uint32_t)(nk - t * S::BK) * (uint32_t)vrow;
  };
  auto plan_fill = [&](int kt, int st) {
    if constexpr (MASK == kMaskBitmask) {
      frk = tile_words(Kb, kt, krow);
      frv = tile_words(Vb, kt, vrow);
    } else {  // kt is the tile above the previous plan's (or < 0)
      ak += ck;
      av += cv;
      nkb -= ck;
      nvb -= cv;
      // Ranges are clamped below 2^31: padding slots read at offset 2^31
      // (kPastEnd), which must stay out of range.
      const bool live = kt >= 0;
      const uint32_t bk = nkb < 0x7FFFFFFFu ? nkb : 0x7FFFFFFFu, bv = nvb < 0x7FFFFFFFu ? nvb : 0x7FFFFFFFu;
      frk = i32x4{(int)(uint32_t)ak, (int)(uint32_t)(ak >> 32), live ? (int)bk : 0, 0x00020000};
      frv = i32x4{(int)(uint32_t)av, (int)(uint32_t)(av >> 32), live ? (int)bv : 0, 0x00020000};
    }
    fst = st;
    fkt = kt;
  };
  auto fill_begin = [&]() {  // the uneven rest of the planned fill
#pragma unroll
    for (int i = FK; i < S::KWIN; ++i) kwin(frk, fst, i);
#pragma unroll
    for (int i = FV; i < S::VWIN; ++i) vwin(frv, fst, i);
    if constexpr (MASK == kMaskBitmask)
      fill_mask(mask_rsrc(fkt < 0 ? 0 : n - q0), fst, fkt < 0 ? 0 : fkt * S::BK);
  };
  auto fill_item = [&](int i) {  // i < FK + FV
    if (i < FK) kwin(frk, fst, i);
    else vwin(frv, fst, i - FK);
  };
  // ---- per-lane LDS read bases (everything else is a constant offset) -----
  // Row operands (S^T, dP^T): A-operand lane m = lane % 32 of a 32-key chunk
  // reads key row perm(m), 16-byte chunk 2 s + hh.
  const int krb = perm(lane & 31) * S::KS + 16 * hh, vrb = perm(lane & 31) * S::VS + 16 * hh;
  // Transposed operand (K^T): lane r of a 16-lane group gives the address of
  // key row hh + 4 (r / 4) (+ 2 for the upper four contraction indices, + 16
  // per key step), columns 32 blk + 16 g1 + 4 (r % 4): it then receives
  // column 32 blk + 16 g1 + r of key rows hh, hh + 4, hh + 8, hh + 12, which
  // are the rows perm() put at C rows 4 hh + 0..3 (resp. 8 + 4 hh + 0..3).
  const int r16 = lane & 15;
  const int ktb = (hh + 4 * (r16 >> 2)) * S::KS + 2 * (16 * g1 + 4 * (r16 & 3));

  // Exponent scale: c log2(e), with c = 0 replaced by 1e-30 (every finite
  // score then maps to exactly exp2(-L log2 e), as for c = 0, while the
  // masking sentinel below still maps to zero).
  const float scale2 = p.scale2 == 0.f ? 1e-30f : p.scale2;
  const float masked_score = scale2 > 0.f ? -INFINITY : INFINITY;  // exp2(score * scale2 - l) = 0
  // Partially allowed tile: scores of disallowed pairs -> the sentinel.
  // Register r of a half holds C row m = 8 (r / 4) + 4 hh + r % 4, i.e. key
  // row 32 c + perm(m) of the tile, for query qa + 32 u.
  auto mask_chunk = [&](f32x16 (&sc)[2], int st, int c, int k0) {
    const uint32_t* ms = reinterpret_cast<const uint32_t*>(mws + st * S::MTILE);
    if constexpr (MASK == kMaskBitmask) {
      if (k0 + S::BK <= nk) {  // every key of the tile exists: the word's bit alone decides
        const uint32_t sentinel = __float_as_uint(masked_score);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t word = ms[(64 * w + 32 * u + (lane & 31)) * S::MWORDS + c];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = perm(8 * (r >> 2) + 4 * hh + (r & 3));
            const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)word, (uint32_t)kk, 1u);
            sc[u][r] = __uint_as_float((__float_as_uint(sc[u][r]) & keep) | (sentinel & ~keep));
          }
        }
        return;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = qa + 32 * u;
      uint32_t word = 0xFFFFFFFFu;
      if constexpr (MASK == kMaskBitmask) word = ms[(64 * w + 32 * u + (lane & 31)) * S::MWORDS + c];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = perm(8 * (r >> 2) + 4 * hh + (r & 3));
        const int key = k0 + 32 * c + kk;
        bool ok = key < nk;
        if constexpr (MASK == kMaskCausal) ok = ok && key <= q + coff;
        if constexpr (MASK == kMaskBitmask) ok = ok && ((word >> kk) & 1u);
        sc[u][r] = ok ? sc[u][r] : masked_score;
      }
    }
  };

  // S^T and dP^T - D of one chunk (32 keys at tile row 32 c) from stage st.
  auto score_products = [&](f32x16 (&sc)[2], f32x16 (&dp)[2], int st, int c) {
    const char* kb = kts + st * S::KTILE + 32 * c * S::KS + krb;
    const char* vb = vts + st * S::VTILE + 32 * c * S::VS + vrb;
#pragma unroll
    for (int s = 0; s < S::NQF; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + 32 * s);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (s == 0) mfma_vz(sc[u], a, qf[u][s]);
        else mfma_vacc(sc[u], a, qf[u][s]);
      }
    }
#pragma unroll
    for (int s = 0; s < S::NVF; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vb + 32 * s);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (s == 0) {
          mfma_vc(dp[u], a, of[u][s], dinit[u]);
        } else {
          mfma_vacc(dp[u], a, of[u][s]);
        }
      }
    }
    nops_after_mfma();
    after_nops_v(sc[0], sc[1], dp[0], dp[1]);
  };

  // One pipeline step for chunk (st, c): sc, dp hold its S^T and dP^T - D
  // (masked); nsc, ndp receive those of the next chunk (stage nst, chunk nc),
  // computed from whatever that stage holds (unused after the last chunk).
  //   phase A: MFMA S^T, dP^T (next chunk)   || VALU P, dS (this chunk)
  //   phase B: MFMA dQ^T (this chunk) with transposed K reads
  // Row operand i of a step's first phase (K, V interleaved) for chunk c of stage st.
  auto is_k = [](int i) { return ((i + 1) * S::NQF) / S::NR > (i * S::NQF) / S::NR; };
  auto arow = [&](int st, int c, int i) -> bf16x8 {
    const int si = (i * S::NQF) / S::NR;
    if (is_k(i)) return *reinterpret_cast<const bf16x8*>(kts + st * S::KTILE + 32 * c * S::KS + krb + 32 * si);
    return *reinterpret_cast<const bf16x8*>(vts + st * S::VTILE + 32 * c * S::VS + vrb + 32 * (i - si));
  };
  // First-phase row operands in flight across steps: a chunk-1 step loads the
  // first kDqPrefetchA operands of the following step (its stage is already
  // visible), which then starts without waiting for them.
  bf16x8 afr[kDqPrefetchA];
  auto step = [&](auto dofill, f32x16 (&sc)[2], f32x16 (&dp)[2], f32x16 (&nsc)[2], f32x16 (&ndp)[2], int st, int c,
                  int nst, int nc, auto hook, auto pre_a, int nkey0) {
    const char* kb = kts + st * S::KTILE + 32 * c * S::KS + ktb;
    // Phase B's transposed K operands; the first PB are read in phase A's last sub-slices.
    auto bread = [&](int j, i16x4& lo, i16x4& hi) {
      const int ks = j / S::NDB, blk = j % S::NDB;
      lo = lds_read_tr(kb + 16 * ks * S::KS, 64 * blk);
      hi = lds_read_tr(kb + (16 * ks + 2) * S::KS, 64 * blk);
    };
    constexpr int PB = kDqPrefetchB;  // transposed operands in flight
    i16x4 tlo[PB], thi[PB];

    // ---- phase A ----
    constexpr int PF = kDqPrefetchA;  // row operands in flight
    auto aread = [&](int i) -> bf16x8 { return arow(nst, nc, i); };  // operand i: K or V, interleaved
    if constexpr (!decltype(pre_a)::value) {
#pragma unroll
      for (int i = 0; i < PF; ++i) afr[i] = aread(i);
    }
    u32x4 sk[2][2];
    // Weights of row pair pr (half pr / 8, registers 2 (pr % 8) and +1) in
    // three stages, so that each exponential's latency is covered by later
    // work: w1 = both exponents and the first exponential, w2 = the second
    // exponential, w3 = dS and the bf16 packing.
    float pt[16], pe[16][2];
    auto w1 = [&](int pr) {
      const int u = pr >> 3, r = 2 * (pr & 7);
      pe[pr][0] = fast_exp2(__builtin_fmaf(sc[u][r], scale2, -l2[u]));
      pt[pr] = __builtin_fmaf(sc[u][r + 1], scale2, -l2[u]);
    };
    auto w2 = [&](int pr) { pe[pr][1] = fast_exp2(pt[pr]); };
    auto w3 = [&](int pr) {
      const int u = pr >> 3, r = 2 * (pr & 7);
      if constexpr (DROP) {  // dp = dP - keep D: keep dS = P (Z ? dp : -keep D)
        const uint32_t m0 = keep_mask(u, r), m1 = keep_mask(u, r + 1);
        const float v0 = __uint_as_float((__float_as_uint(dp[u][r]) & m0) | (__float_as_uint(dn[u]) & ~m0));
        const float v1 = __uint_as_float((__float_as_uint(dp[u][r + 1]) & m1) | (__float_as_uint(dn[u]) & ~m1));
        sk[u][r >> 3][(r >> 1) & 3] = pack_bf16x2(pe[pr][0] * v0, pe[pr][1] * v1);
      } else {
        sk[u][r >> 3][(r >> 1) & 3] = pack_bf16x2(pe[pr][0] * dp[u][r], pe[pr][1] * dp[u][r + 1]);
      }
    };
    // Work items in issue order: w1(k), w2(k), w3(k - 1) for k = 0..15, then
    // w3(15); item t goes to sub-slice t * NSUB / NITEM.
    constexpr int NSUB = 2 * S::NR, NITEM = 3 * 16;
    auto item = [&](int t) {
      const int k = t / 3, st3 = t % 3;
      if (st3 == 0) w1(k);
      else if (st3 == 1) w2(k);
      else if (k > 0) w3(k - 1);
    };
    // Sub-slice m: one MFMA (operand m / 2, half m % 2) and its share of the
    // vector work; the second sub-slice of an operand issues the prefetch
    // read, every fourth sub-slice one tile copy.
#pragma unroll
    for (int m = 0; m < NSUB; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = m / 2, u = m % 2;
      const int si = (i * S::NQF) / S::NR;
      if (is_k(i)) {
        if (si == 0) mfma_vz(nsc[u], afr[i % PF], qf[u][si]);
        else mfma_vacc(nsc[u], afr[i % PF], qf[u][si]);
      } else {
        const int vi = i - si;
        if (vi == 0) {
          mfma_vc(ndp[u], afr[i % PF], of[u][vi], dinit[u]);
        } else {
          mfma_vacc(ndp[u], afr[i % PF], of[u][vi]);
        }
      }
      if (u == 1 && i + PF < S::NR) afr[i % PF] = aread(i + PF);
      if (u == 1 && i >= S::NR - PB) bread(i - (S::NR - PB), tlo[i - (S::NR - PB)], thi[i - (S::NR - PB)]);
      if constexpr (decltype(dofill)::value) {
        if (m % 4 == 1 && m / 4 < FK + FV) fill_item(m / 4);
      }
#pragma unroll
      for (int t = (m * NITEM + NSUB - 1) / NSUB; t < ((m + 1) * NITEM + NSUB - 1) / NSUB; ++t) item(t);
    }
    __builtin_amdgcn_sched_barrier(0);
    w3(15);
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase B ----
    // Operand j: key step j / NDB, column block j % NDB; two MFMAs (halves).
    if constexpr (DROP) draw_init(nkey0);
    asm volatile("s_nop 1");  // the last packed dS operands were just written
    // Slice j: two MFMAs (halves) and the reads PB operands ahead.
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      const int ks = j / S::NDB, blk = j % S::NDB;
      const bf16x8 a = join_tr(tlo[j % PB], thi[j % PB]);
#pragma unroll
      for (int u = 0; u < 2; ++u)  // (64, 64): the allocator moves accumulators through VGPRs
        mfma_aacc_g<D == 64 && DV == 64>(dq[u][blk], a, __builtin_bit_cast(bf16x8, sk[u][ks]));
      if (j + PB < S::NB) bread(j + PB, tlo[j % PB], thi[j % PB]);
      if (j == 2) hook();
      if constexpr (decltype(dofill)::value) {  // chunk 1: the next step's first row operands
        if (j >= S::NB - PF) afr[j - (S::NB - PF)] = arow(nst, 1, j - (S::NB - PF));
      }
      if constexpr (DROP) {  // the next chunk's two calls: 28 items over the NB slices
#pragma unroll
        for (int t = j * 28 / S::NB; t < (j + 1) * 28 / S::NB; ++t) draw_item(t);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DROP) draw_share();
  };

  // ---- main loop -------------------------------------------------------------
  // This split's share of the key tiles [0, kt_end): [t0, kt_end).
  int t0 = 0;
  if (p.dq_splits > 1) {
    const int per = (kt_end + p.dq_splits - 1) / p.dq_splits;
    t0 = split * per < kt_end ? split * per : kt_end;
    kt_end = t0 + per < kt_end ? t0 + per : kt_end;
  }
  if (MASK == kMaskBitmask) {
    __syncthreads();  // tile classes staged
    if (t0 < kt_end && tile_class(t0) == kTileEmpty) t0 = next_tile(t0);
  }
  if (t0 >= kt_end) t0 = -1;
  int t1 = next_tile(t0), t2 = next_tile(t1), t3 = next_tile(t2);
  int ntiles = 0;
  if (t0 >= 0) {  // workgroup-uniform
    fill(t0, 0);
    fill(t1, 1);
    fill(t2, 2);
    if constexpr (MASK != kMaskBitmask) plan_start(t2);
    wait_vm_n<2 * kF>();
    __syncthreads();
    f32x16 sa[2], pa[2], sb[2], pb[2];
    score_products(sa, pa, 0, 0);
    if constexpr (DROP) {  // the first chunk's calls
      draw_init(t0 * S::BK);
#pragma unroll
      for (int t = 0; t < 28; ++t) draw_item(t);
      draw_share();
    }
#pragma unroll
    for (int i = 0; i < kDqPrefetchA; ++i) afr[i] = arow(0, 1, i);  // the first step's first operands
    unsigned j = 0;  // position of t0 in the sequence; its stage is j % NSTAGE
    while (true) {
      const int st = (int)(j & (S::NSTAGE - 1)), nst = (int)((j + 1) & (S::NSTAGE - 1));
      const int k0 = t0 * S::BK;
      const bool partial = tile_partial(t0);
      // chunk 0 of t0
      if (partial) mask_chunk(sa, st, 0, k0);
      step(std::false_type{}, sa, pa, sb, pb, st, 0, st, 1,
           [&] { plan_fill(t3, (int)((j + 3) & (S::NSTAGE - 1))); }, std::true_type{}, k0 + 32);
      // The next tile's stage must be complete and visible before chunk 1's
      // phase A reads it; after this barrier every wave is past tile j-1, so
      // its stage takes the fill of position j+3 (empty past the last tile),
      // spread over chunk 1's first phase.
      wait_vm_n<kF>();
      __syncthreads();
      fill_begin();
      // chunk 1 of t0
      if (partial) mask_chunk(sb, st, 1, k0);
      step(std::true_type{}, sb, pb, sa, pa, st, 1, nst, 0, [] {}, std::false_type{}, t1 < 0 ? 0 : t1 * S::BK);
      ++ntiles;
      if (t1 < 0) break;
      t0 = t1;
      t1 = t2;
      t2 = t3;
      t3 = next_tile(t2);
      ++j;
    }
    nops_after_mfma();  // the last dQ^T products were just issued
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < S::NDB; ++i) after_nops_a(dq[u][i]);
    wait_vm_n<0>();  // copies of empty positions
  }
  count_tiles(p.tile_count_dq, ntiles);

  if constexpr (DROP) {  // the 1 / keep of dS
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < S::NDB; ++i) dq[u][i] *= p.drop.keep_inv;
  }
  if (p.dq_splits > 1) {  // this split's unscaled fp32 partial, for bwd_dq_merge_kernel
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = qa + 32 * u;
      if (q < n) {
        float* part = p.dQpart + (((int64_t)split * p.B * p.H + unit) * n + q) * D;
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c0 = db * 32 + 8 * g + 4 * hh;
            *reinterpret_cast<f32x4*>(part + c0) =
                f32x4{dq[u][db][4 * g], dq[u][db][4 * g + 1], dq[u][db][4 * g + 2], dq[u][db][4 * g + 3]};
          }
      }
    }
    return;
  }
  // Epilogue: dQ = c dQ^T (lane = query; 4 consecutive columns per store).
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = qa + 32 * u;
    if (q < n) {
      char* dQp = (char*)p.dQ + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1] + (int64_t)q * p.sq[2]) * 2;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = db * 32 + 8 * g + 4 * hh;
          const float x0 = dq[u][db][4 * g] * p.scale, x1 = dq[u][db][4 * g + 1] * p.scale;
          const float x2 = dq[u][db][4 * g + 2] * p.scale, x3 = dq[u][db][4 * g + 3] * p.scale;
          *reinterpret_cast<u32x2*>(dQp + c0 * 2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
    }
  }
}

template <int D, int DV, int MASK>
static int launch_dq_pipe(const BwdParams& p, hipStream_t st) {
  if (p.drop.p8 != 0)
    hipLaunchKernelGGL((bwd_dq_pipe_kernel<D, DV, MASK, true>), dim3((unsigned)p.grid_pad_dq), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_dq_pipe_kernel<D, DV, MASK, false>), dim3((unsigned)p.grid_pad_dq), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

template <int D, int DV>
static int launch_dq_pipe_mask(const BwdParams& p, int mask_mode, hipStream_t st) {
  switch (mask_mode) {
    case kMaskNone: return launch_dq_pipe<D, DV, kMaskNone>(p, st);
    case kMaskCausal: return launch_dq_pipe<D, DV, kMaskCausal>(p, st);
    default: return launch_dq_pipe<D, DV, kMaskBitmask>(p, st);
  }
}

// Sum of the key-range splits' partial dQ, in split order (so the result is
// reproducible bit for bit), times c, converted to bf16.  One thread per
// (row, 4 columns).
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_merge_kernel(BwdParams p) {
  const int64_t rows = (int64_t)p.B * p.H * p.n;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (D / 4)) return;
  const int64_t row = t / (D / 4);
  const int c4 = (int)(t % (D / 4));
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.dq_splits; ++s) acc += *reinterpret_cast<const f32x4*>(p.dQpart + (s * rows + row) * D + 4 * c4);
  const int64_t unit = row / p.n, i = row % p.n;
  const int64_t b = unit / p.H, h = unit % p.H;
  const int64_t off = b * p.sq[0] + h * p.sq[1] + i * p.sq[2] + 4 * c4;
  *reinterpret_cast<u32x2*>((char*)p.dQ + off * 2) =
      u32x2{pack_bf16x2(acc[0] * p.scale, acc[1] * p.scale), pack_bf16x2(acc[2] * p.scale, acc[3] * p.scale)};
}

int launch_bwd_dq_merge(const BwdParams& p, int d, void* stream) {
  const int64_t threads = (int64_t)p.B * p.H * p.n * (d / 4);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  hipStream_t st = (hipStream_t)stream;
  if (d == 128) hipLaunchKernelGGL((bwd_dq_merge_kernel<128>), grid, block, 0, st, p);
  else if (d == 64) hipLaunchKernelGGL((bwd_dq_merge_kernel<64>), grid, block, 0, st, p);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_bwd_dq_pipe(const BwdParams& p, int d, int v, int mask_mode, void* stream) {
  static_assert(DqPipeShape<128, 128>::MAXTK == kDqPipeMaxTk, "staged tile classes");
  hipStream_t st = (hipStream_t)stream;
  if (d == 128 && v == 128) return launch_dq_pipe_mask<128, 128>(p, mask_mode, st);
  if (d == 64 && v == 128) return launch_dq_pipe_mask<64, 128>(p, mask_mode, st);
  if (d == 64 && v == 64) return launch_dq_pipe_mask<64, 64>(p, mask_mode, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace eta
