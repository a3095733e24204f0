// Backward, key-tile-outer dK / dV kernel for bf16 with (d, v) = (128, 128), (64, 128) or (64, 64):
// the main kernel of the deterministic backward (dQ comes from the
// query-tile-outer kernel).
//
// Method (alphabetamath page, reverse procedure; ob1 page, part 2;
// HarshvardhanJ README, backward section): with the forward's L and
// D_i = <dO_i, O_i>, for each block recompute s_ij = c <Q_i, K_j>,
// p_ij = exp(s_ij - L_i), dP_ij = <dO_i, V_j>, dS_ij = p_ij (dP_ij - D_i), and
// accumulate dV_j += p_ij dO_i, dK_j += c dS_ij Q_i.  Tiles whose intersection
// with every row's allowed set is empty are skipped; only partially allowed
// tiles are masked (ob1 page, part 3).
//
// gfx950 design.  One workgroup (one per CU) owns 128 keys, 32 per wave; a
// wave keeps its K and V rows in AGPRs as MFMA B operands and its dK^T,
// dV^T accumulators in AGPRs for the whole loop over query tiles, while the
// S / dP accumulators live in VGPRs, where the vector ALUs read them without
// copies, and each dP accumulator starts from -D, so that dS = P (dP - D) is
// one multiply (explicit-register MFMAs of kern_common.h; their wait states are
// kept by construction: scores are read one 16-MFMA phase after they are
// written, s_nop after the prologue's products and before the epilogue, the
// packed P / dS operands written before the second phase's first read).  Query tiles of 64
// rows are visited from the last one down and processed as two chunks of 32
// rows.  Per chunk, S = Q K^T and dP = dO V^T put one key in each lane
// column, so the registers holding P and dS are directly the B operand of
// dV^T += dO^T P and dK^T += Q^T dS, whose dO^T / Q^T operands come from the
// row-major tiles through transposed LDS reads.  The chunks form a software
// pipeline: the S / dP products of chunk k+1 run on the matrix cores while
// the vector ALUs turn chunk k's scores into P and dS, then chunk k's dV / dK
// products run; the instruction order is pinned with scheduling barriers.
// Q, dO, L log2(e) and D (and the bitmask words) are copied from HBM
// straight into a 4-stage ring of LDS tiles (buffer_load ... lds, issued
// from inline assembly and counted with vmcnt), two tiles ahead of their
// use, with one barrier per tile.  Tile rows are padded by 16 bytes and the
// query rows of each group of 16 are taken in transposed order (4 u + v ->
// u + 4 v) by the score products, so the transposed reads of dO^T and Q^T
// cover rows 4 apart: both kinds of read are then free of bank conflicts
// and every LDS read address is one per-lane register plus a constant.
//
// Dropout (DROP; alphabetamath page, reverse procedure, closing remark: the
// reverse pass replays the forward's realised mask): with keep decisions Z
// and keep = P(kept), dV^T += dO^T (P o Z) and keep dS = P (Z dP - keep D)
// (both times 1 / keep at the end): the dP accumulators start from the
// stored -keep D, and a dropped pair takes -keep D instead of dP.  The
// decisions are the counter-based draws of kern_common.h, regenerated: the
// chunk's 32 rows form 8 row blocks of 4, a lane's key one key block of 4
// with its quad, so the 8 lanes sharing a key block (a quad in each half)
// draw the chunk's 8 calls, one each, in the previous step's second phase
// (where the vector ALUs are idle), and exchange them by one half swap and
// quad broadcasts.
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {
#ifndef ETA_KV_PREFETCH_A
#define ETA_KV_PREFETCH_A 4
#endif
#ifndef ETA_KV_PREFETCH_B
#define ETA_KV_PREFETCH_B 3
#endif
// LDS operand prefetch depth, in MFMAs, of the two phases.
constexpr int kPrefetchA = ETA_KV_PREFETCH_A, kPrefetchB = ETA_KV_PREFETCH_B;

template <int D, int DV>
struct KvShape {
  static constexpr int NW = 4;
  static constexpr int BK = kBwdBk;  // keys per workgroup, 32 per wave
  static constexpr int BQ = kBwdBq;  // queries per tile: two chunks of 32
  static constexpr int NSTAGE = 4;   // LDS ring: tiles j .. j+2 resident or in flight
  static_assert((NSTAGE & (NSTAGE - 1)) == 0, "power-of-two ring");
  static constexpr int NQF = D / 16, NVF = DV / 16;  // K / V fragments per lane
  static constexpr int NDB = D / 32, NVB = DV / 32;  // 32-column blocks of dK^T / dV^T
  static constexpr int NA = NQF + NVF;               // S and dP MFMAs per chunk
  static constexpr int NB = 2 * (NDB + NVB);         // dK and dV MFMAs per chunk
  using QT = PadTile<D * 2, 16>;
  using OT = PadTile<DV * 2, 16>;
  static constexpr int QS = QT::kStride, OS = OT::kStride;
  static constexpr int QTILE = BQ * QS, OTILE = BQ * OS;
  static constexpr int QWINS = QTILE / 1024, OWINS = OTILE / 1024;  // 1 KB fill windows per tile
  // Copies per wave and tile (QWIN / OWIN): a contiguous run of windows, the
  // last of which is an empty copy for some waves.
  static constexpr int QWIN = (QWINS + NW - 1) / NW, OWIN = (OWINS + NW - 1) / NW;
  static constexpr int MWORDS = BK / 32;
  // Per stage: L log2(e) [BQ], D [BQ], mask words [BQ][MWORDS].
  static constexpr int LD_L = 0, LD_D = BQ * 4, LD_M = 2 * BQ * 4;
  static constexpr int LDB = LD_M + BQ * MWORDS * 4;
  static constexpr int MAXTQ = 4096;  // bitmask: query tiles whose classes are staged in LDS
  static_assert(QTILE % 1024 == 0 && OTILE % 1024 == 0, "whole fill windows");
  static_assert(BQ == 64 && BK == 128, "two chunks of 32 queries, 32 keys per wave");
};

template <int D, int DV, int MASK, bool DROP>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(BwdParams p) {
  using S = KvShape<D, DV>;
  __shared__ __attribute__((aligned(1024))) char qs[S::NSTAGE * S::QTILE];
  __shared__ __attribute__((aligned(1024))) char os[S::NSTAGE * S::OTILE];
  __shared__ __attribute__((aligned(16))) char lds_ld[S::NSTAGE * S::LDB];
  __shared__ uint8_t cls_s[MASK == kMaskBitmask ? S::MAXTQ : 1];
  __shared__ __attribute__((aligned(1024))) char spare[4096];  // target of the padding copies (any immediate offset)

  const int64_t logical = xcd_logical(blockIdx.x, p.grid_pad, p.total);
  if (logical < 0) return;
  const int unit = (int)(logical / p.tk);
  const int kt = (int)(logical % p.tk);  // low key tiles (most causal work) first
  const int b = unit / p.H, h = unit % p.H;
  const int n = (int)p.n, nk = (int)p.nk, coff = (int)p.coff;  // query rows, key rows, causal offset
  const int k0 = kt * S::BK;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int g1 = (lane >> 4) & 1;
  const int klocal = 32 * w + (lane & 31);
  const int key = k0 + klocal;
  const bool kvalid = key < nk;

  const int qrow = (int)p.sq[2] * 2, krow = (int)p.sk[2] * 2;
  const int vrow = (int)p.sv[2] * 2, orow = (int)p.so[2] * 2;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * 2;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * 2;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * 2;
  const char* dOb = (const char*)p.dO + ((int64_t)b * p.so[0] + (int64_t)h * p.so[1]) * 2;
  const float* L2b = p.L2 + (int64_t)unit * p.n_pad;
  const float* Dnb = p.Dn + (int64_t)unit * p.n_pad;
  const uint32_t* mbase = nullptr;
  if constexpr (MASK == kMaskBitmask) mbase = p.mask + b * p.mask_sb + h * p.mask_sh;

  // Clear the ring once when the last query tile is partial: tile rows that a
  // fill leaves untouched (past n) then always hold finite values.  With n a
  // multiple of the tile height every fill writes every row the kernel reads
  // (row pads are never read), so short workgroups skip the 34 stores per
  // thread.
  if (n % S::BQ != 0) {
    for (int c = tid; c < S::NSTAGE * S::QTILE / 16; c += 256) reinterpret_cast<u32x4*>(qs)[c] = u32x4{0, 0, 0, 0};
    for (int c = tid; c < S::NSTAGE * S::OTILE / 16; c += 256) reinterpret_cast<u32x4*>(os)[c] = u32x4{0, 0, 0, 0};
    for (int c = tid; c < S::NSTAGE * S::LDB / 16; c += 256) reinterpret_cast<u32x4*>(lds_ld)[c] = u32x4{0, 0, 0, 0};
  }

  // Query-tile sequence: from the last tile down to the first that can hold
  // an allowed pair (causal: the tile containing row k0 - coff); bitmask tiles come
  // from the tile map, staged in LDS so that the loop issues no loads of its own.
  int qt_first = 0;
  if constexpr (MASK == kMaskCausal) {
    // Row k0 - coff is the first that allows key k0.  Past the last row no
    // query tile holds an allowed pair: the tile containing that padding row
    // is empty, not partial, and must not be visited.
    const int r0 = k0 - coff;
    qt_first = r0 >= n ? p.tq : (r0 > 0 ? r0 / S::BQ : 0);
  }
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    const uint8_t* map_col = p.map + mu * (int64_t)p.tq * p.tk + kt;
    for (int t = tid; t < p.tq; t += 256) cls_s[t] = map_col[(int64_t)t * p.tk];
  }
  auto tile_class = [&](int qt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return cls_s[qt];
    return classify_analytic(MASK, (int64_t)qt * S::BQ, S::BQ, k0, S::BK, n, nk, coff);
  };
  // Partially allowed among the visited (nonempty) tiles, with 32-bit scalar
  // arithmetic: causal tiles from row t_full on are full when every key of
  // the tile exists.
  const bool keys_whole = k0 + S::BK <= nk;
  int t_full = 0;
  if constexpr (MASK == kMaskCausal) {
    const int r_full = k0 + S::BK - 1 - coff;  // first query row that allows every key of the tile
    t_full = r_full <= 0 ? 0 : (r_full + S::BQ - 1) / S::BQ;
  }
  auto tile_partial = [&](int qt) -> bool {
    if constexpr (MASK == kMaskBitmask) return cls_s[qt] == kTilePartial;
    if constexpr (MASK == kMaskCausal) return !(keys_whole && qt >= t_full);
    return !keys_whole;
  };
  auto next_tile = [&](int qt) -> int {  // next (lower) tile with an allowed pair, or -1
    if (qt < 0) return -1;
    if constexpr (MASK != kMaskBitmask) return qt - 1 >= qt_first ? qt - 1 : -1;
    for (int t = qt - 1; t >= 0; --t)
      if (tile_class(t) != kTileEmpty) return t;
    return -1;
  };

  // K and V rows of this wave's keys (B operands; lane column = key).
  bf16x8 kf[S::NQF], vf[S::NVF];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb, (int64_t)nk * krow);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vb, (int64_t)nk * vrow);
#pragma unroll
    for (int s = 0; s < S::NQF; ++s)
      kf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, key * krow + (16 * s + 8 * hh) * 2, 0, 0));
#pragma unroll
    for (int s = 0; s < S::NVF; ++s)
      vf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, key * vrow + (16 * s + 8 * hh) * 2, 0, 0));
  }
  f32x16 dk[S::NDB], dv[S::NVB];
#pragma unroll
  for (int i = 0; i < S::NDB; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < S::NVB; ++i) dv[i] = f32x16{};

  // ---- tile fills ----------------------------------------------------------
  // Wave w copies a contiguous run of 1 KB windows of each tile: QB = QWINS /
  // NW of them, plus one more for the first QX = QWINS % NW waves (the others
  // issue that item as an empty copy into the spare window, so that every
  // wave issues the same instructions).  Consecutive windows share one M0
  // value in groups of four: the copy's immediate offset selects the window
  // and is taken off the per-lane source offsets.
  constexpr int QB = S::QWINS / S::NW, QX = S::QWINS % S::NW;
  constexpr int OB = S::OWINS / S::NW, OX = S::OWINS % S::NW;
  static_assert(S::QWIN == QB + (QX > 0) && S::OWIN == OB + (OX > 0), "window counts");
  const int qfirst = w * QB + (w < QX ? w : QX), ofirst = w * OB + (w < OX ? w : OX);
  int qsrc[S::QWIN], osrc[S::OWIN];
#pragma unroll
  for (int i = 0; i < S::QWIN; ++i)
    qsrc[i] = (int)((uint32_t)S::QT::fill_src((qfirst + i) * 1024 + 16 * lane, qrow) - (uint32_t)((i % 4) * 1024));
#pragma unroll
  for (int i = 0; i < S::OWIN; ++i)
    osrc[i] = (int)((uint32_t)S::OT::fill_src((ofirst + i) * 1024 + 16 * lane, orow) - (uint32_t)((i % 4) * 1024));
  // Query row of the tile behind LDS slot l of the L / D copies (and behind
  // lane l % 32 of a score product's A operand): groups of 16 rows taken in
  // transposed order, 4 u + v -> u + 4 v.
  auto perm = [](int l) { return (l & ~15) + ((l & 15) >> 2) + 4 * (l & 3); };
  const uint32_t qs_l = lds_address(qs), os_l = lds_address(os), ld_l = lds_address(lds_ld);
  const uint32_t sp_l = lds_address(spare);
  // Per tile every wave issues QWIN + OWIN tile copies, one row copy (L
  // log2(e) rows by wave 0, -D rows by wave 1, empty ranges by the others)
  // and, with a bitmask, one more (mask words of 16 query rows).
  constexpr int kBm = MASK == kMaskBitmask;
  constexpr int kF = S::QWIN + S::OWIN + 1 + kBm;
  const i32x4 r_none = rsrc_words(Qb, 0);
  // Item i of this wave's run over a tile at LDS byte address `tile`.
  auto win_item = [&](const i32x4& r, uint32_t tile, int first, int nb, int nx, const auto& src, int i) {
    const bool extra = i == nb;
    const bool real = !extra || w < nx;
    if (i % 4 == 0 || extra)  // group start, or the item that may be an empty copy
      set_m0(real ? tile + (first + 4 * (i / 4)) * 1024 : sp_l);  // an empty copy lands at sp_l + (i % 4) KB
    // An empty copy keeps the resource's address and takes an empty range.
    fill16_off(i32x4{r[0], r[1], real ? r[2] : 0, r[3]}, src[i], i % 4);
  };
  auto qwin = [&](const i32x4& rq, int st, int i) { win_item(rq, qs_l + st * S::QTILE, qfirst, QB, QX, qsrc, i); };
  auto owin = [&](const i32x4& ro, int st, int i) { win_item(ro, os_l + st * S::OTILE, ofirst, OB, OX, osrc, i); };
  // The rest of a tile's copies (row statistics, mask words); qt < 0 copies
  // nothing (empty buffer ranges) but issues the same instructions.
  auto fill_mask = [&](int qt, int st) {
    if constexpr (MASK == kMaskBitmask) {
      // Row 16 w + lane / 4 of the tile, word lane % 4 of this key tile.
      const int q0 = qt < 0 ? 0 : qt * S::BQ;
      const int r = 16 * w + lane / 4;
      const i32x4 rm = rsrc_words(mbase + (int64_t)q0 * p.mask_si, qt < 0 ? 0 : (int64_t)(n - q0) * p.mask_si * 4);
      fill4(rm, ld_l + st * S::LDB + S::LD_M + 256 * w, (int)(((int64_t)r * p.mask_si + (k0 >> 5) + (lane & 3)) * 4));
    }
  };
  auto fill_rows = [&](int qt, int st) {
    const int q0 = qt < 0 ? 0 : qt * S::BQ;
    const bool rows_real = w < 2 && qt >= 0;  // padded rows: always in range; slot l holds row perm(l)
    const float* src = (w == 0 ? L2b : Dnb) + q0;
    fill4(rows_real ? rsrc_words(src, S::BQ * 4) : r_none,
          w < 2 ? ld_l + st * S::LDB + (w == 0 ? S::LD_L : S::LD_D) : sp_l, 4 * perm(lane));
    fill_mask(qt, st);
  };
  auto fill = [&](int qt, int st) {
    const int q0 = qt < 0 ? 0 : qt * S::BQ;
    const int64_t rows = qt < 0 ? 0 : n - q0;
    const i32x4 rq = rsrc_words(Qb + (int64_t)q0 * qrow, rows * qrow);
    const i32x4 ro = rsrc_words(dOb + (int64_t)q0 * orow, rows * orow);
#pragma unroll
    for (int i = 0; i < S::QWIN; ++i) qwin(rq, st, i);
#pragma unroll
    for (int i = 0; i < S::OWIN; ++i) owin(ro, st, i);
    fill_rows(qt, st);
  };
  // The same copies split in two, for the fill issued inside a pipeline step:
  // the first FQ + FO items (issued one per MFMA of chunk 1's first phase)
  // and the rest (the extra items, rows, mask words), issued right after the
  // mid-tile barrier.  Their buffer resources are computed by plan_fill in
  // chunk 0's second phase, where the scalar work issues under the MFMAs.
  constexpr int FQ = QB, FO = OB;
  // Buffer resource of the rows of query tile q0.. of a [n, row] slice with
  // rb bytes per row; the host bounds (n - 1) rb + the row width by 2^31 - 1,
  // so the products below fit in 32 bits.  qt < 0: an empty range.
  auto tile_words = [&](const void* base, int qt, int rb) -> i32x4 {
    const uint32_t q0 = qt < 0 ? 0u : (uint32_t)(qt * S::BQ);
    const uint32_t nb = qt < 0 ? 0u : (uint32_t)(n - (int)q0) * (uint32_t)rb;
    const uint64_t a = reinterpret_cast<uint64_t>(base) + q0 * (uint32_t)rb;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)(nb < 0x7FFFFFFFu ? nb : 0x7FFFFFFFu), 0x00020000};
  };
  // The next in-step fill: resources of the Q, dO and row-statistic copies,
  // the query tile and the target stage.
  i32x4 frq, fro, frr;
  int fst = 0, fqt = -1;
  // Without a bitmask the visited query tiles are consecutive (descending):
  // the next fill's resources follow from the previous ones by one tile's
  // bytes (a few scalar instructions per tile instead of a product and a
  // clamp per tensor).  aq / ao / al are the byte addresses of the planned
  // tile's Q, dO and row-statistic rows, nq / no the Q and dO bytes from
  // there to row n (unsigned and unclamped: the host bounds (n - 1) rb + the
  // row width by 2^31 - 1, so they stay below 2^32; the resources take them
  // clamped); a planned tile below 0 gets empty ranges, so its address (then
  // below the tensor) is never used.
  uint64_t aq = 0, ao = 0, al = 0;
  uint32_t nq = 0, no = 0;
  const uint32_t cq = (uint32_t)(S::BQ * qrow), co = (uint32_t)(S::BQ * orow);
  const uint32_t nl = w < 2 ? (uint32_t)(S::BQ * 4) : 0u;  // row statistics: waves 0 (L) and 1 (D)
  auto plan_start = [&](int qt) {  // state of tile qt (any value; qt < 0 only ever precedes empty fills)
    const int q = qt < 0 ? 0 : qt;
    aq = reinterpret_cast<uint64_t>(Qb) + (uint64_t)((uint32_t)q * cq);
    ao = reinterpret_cast<uint64_t>(dOb) + (uint64_t)((uint32_t)q * co);
    al = reinterpret_cast<uint64_t>(w == 0 ? L2b : Dnb) + (uint64_t)q * (S::BQ * 4);
    nq = (uint32_t)(n - q * S::BQ) * (uint32_t)qrow;
    no = (uint32_t)(n - q * S::BQ) * (uint32_t)orow;
  };
  auto rsrc_at = [](uint64_t a, uint32_t nb) -> i32x4 {
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)nb, 0x00020000};
  };
  auto plan_fill = [&](int qt, int st) {
    if constexpr (MASK == kMaskBitmask) {
      frq = tile_words(Qb, qt, qrow);
      fro = tile_words(dOb, qt, orow);
      const float* src = (w == 0 ? L2b : Dnb) + (qt < 0 ? 0 : qt * S::BQ);
      frr = (w < 2 && qt >= 0) ? rsrc_words(src, S::BQ * 4) : r_none;
    } else {  // qt is the tile below the previous plan's (or < 0)
      aq -= cq;
      ao -= co;
      al -= S::BQ * 4;
      nq += cq;
      no += co;
      // Ranges are clamped below 2^31: padding slots read at offset 2^31
      // (kPastEnd), which must stay out of range.
      const bool live = qt >= 0;
      frq = rsrc_at(aq, live ? (nq < 0x7FFFFFFFu ? nq : 0x7FFFFFFFu) : 0u);
      fro = rsrc_at(ao, live ? (no < 0x7FFFFFFFu ? no : 0x7FFFFFFFu) : 0u);
      frr = rsrc_at(al, live ? nl : 0u);
    }
    fst = st;
    fqt = qt;
  };
  auto fill_begin = [&]() {
#pragma unroll
    for (int i = FQ; i < S::QWIN; ++i) qwin(frq, fst, i);
#pragma unroll
    for (int i = FO; i < S::OWIN; ++i) owin(fro, fst, i);
    fill4(frr, w < 2 ? ld_l + fst * S::LDB + (w == 0 ? S::LD_L : S::LD_D) : sp_l, 4 * perm(lane));
    fill_mask(fqt, fst);
  };
  auto fill_item = [&](int i) {  // i < FQ + FO
    if (i < FQ) qwin(frq, fst, i);
    else owin(fro, fst, i - FQ);
  };
  static_assert(FQ + FO <= S::NQF + S::NVF, "one spread fill per first-phase MFMA at most");

  // ---- per-lane LDS read bases (everything else is a constant offset) -----
  // Row operands (S, dP): A-operand lane m = lane % 32 of a 32-row chunk
  // reads row perm(m), 16-byte chunk 2 ks + hh.
  const int qrb = perm(lane & 31) * S::QS + 16 * hh, orb = perm(lane & 31) * S::OS + 16 * hh;
  // Transposed operands (dK, dV): lane r of a 16-lane group gives the address
  // of row hh + 4 (r / 4) (+ 2 for the upper four contraction indices, + 16
  // per key step), columns 32 blk + 16 g1 + 4 (r % 4): it then receives
  // column 32 blk + 16 g1 + r of rows hh, hh + 4, hh + 8, hh + 12, which are
  // the query rows perm() put at C rows 4 hh + 0..3 (resp. 8 + 4 hh + 0..3).
  const int r16 = lane & 15;
  const int qtb = (hh + 4 * (r16 >> 2)) * S::QS + 2 * (16 * g1 + 4 * (r16 & 3));
  const int otb = (hh + 4 * (r16 >> 2)) * S::OS + 2 * (16 * g1 + 4 * (r16 & 3));

  // S and dP of one chunk (32 query rows at tile row 32 c) from stage st.
  auto score_products = [&](f32x16& sc, f32x16& dp, int st, int c, const f32x16& dn) {
    const char* qb = qs + st * S::QTILE + 32 * c * S::QS;
    const char* ob = os + st * S::OTILE + 32 * c * S::OS;
#pragma unroll
    for (int s = 0; s < S::NQF; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qb + qrb + 32 * s);
      if (s == 0) mfma_vz(sc, a, kf[s]);
      else mfma_vacc(sc, a, kf[s]);
    }
#pragma unroll
    for (int s = 0; s < S::NVF; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(ob + orb + 32 * s);
      if (s == 0) {
        mfma_vc(dp, a, vf[s], dn);
      } else {
        mfma_vacc(dp, a, vf[s]);
      }
    }
    nops_after_mfma();
    after_nops_v(sc, dp);
    asm volatile("" ::"v"(dn));  // keep the init registers until its product is done
  };
  // -D of a 32-row chunk of stage st, in the C layout of the dP accumulator
  // (register r holds row 8 (r / 4) + 4 hh + r % 4 of the chunk).
  auto load_dn = [&](int st, int c) -> f32x16 {
    const float* ds = reinterpret_cast<const float*>(lds_ld + st * S::LDB + S::LD_D) + 32 * c + 4 * hh;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(ds), a1 = *reinterpret_cast<const f32x4*>(ds + 8);
    const f32x4 a2 = *reinterpret_cast<const f32x4*>(ds + 16), a3 = *reinterpret_cast<const f32x4*>(ds + 24);
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    const f32x8 lo = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    const f32x8 hi = __builtin_shufflevector(a2, a3, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  };
  // Exponent scale: c log2(e), with c = 0 replaced by 1e-30 (every finite
  // score then maps to exactly exp2(-L log2 e), as for c = 0, while the
  // masking sentinel below still maps to zero).
  const float scale2 = p.scale2 == 0.f ? 1e-30f : p.scale2;
  const float masked_score = scale2 > 0.f ? -INFINITY : INFINITY;  // exp2(score * scale2 - l) = 0
  // Partially allowed tile: scores of disallowed pairs -> the sentinel.
  // Register r of a chunk holds C row m = 8 (r / 4) + 4 hh + r % 4, i.e.
  // query row 32 c + perm(m) of the tile.
  auto mask_chunk = [&](f32x16& sc, int st, int c, int q0) {
    const uint32_t* ms = reinterpret_cast<const uint32_t*>(lds_ld + st * S::LDB + S::LD_M);
    if constexpr (MASK == kMaskBitmask) {
      if (k0 + S::BK <= nk) {  // every key of the tile exists: the word's bit alone decides
        const uint32_t sentinel = __float_as_uint(masked_score);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * c + perm(8 * (r >> 2) + 4 * hh + (r & 3));
          const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)ms[ql * S::MWORDS + w], (uint32_t)(lane & 31), 1u);
          sc[r] = __uint_as_float((__float_as_uint(sc[r]) & keep) | (sentinel & ~keep));
        }
        return;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = 32 * c + perm(8 * (r >> 2) + 4 * hh + (r & 3));
      bool ok = kvalid;
      if constexpr (MASK == kMaskCausal) ok = ok && key <= q0 + ql + coff;
      // The word is read by every lane (the stage always holds the tile's words) and
      // combined without short-circuit, so the 16 reads issue together, not as 16
      // branches that each wait for their own read.
      if constexpr (MASK == kMaskBitmask) ok = ok & (((ms[ql * S::MWORDS + w] >> (lane & 31)) & 1u) != 0u);
      sc[r] = ok ? sc[r] : masked_score;
    }
  };

  // Dropout draws.  Lane (hh, quad position e) draws row block 4 hh + e of a
  // chunk for its quad's key block: counter (key / 4, row / 4, unit, 0).  The
  // call's 16 keep bits are packed as bit 8 (key % 4) + 4 + row % 4.  Register r
  // = 4 g + e' of a chunk holds row 16 (g / 2) + 2 (g % 2) + hh + 4 e' (the
  // perm() order), i.e. row block 4 (g / 2) + e', row 2 (g % 2) + hh in it:
  // the call of the lane in half g / 2 at quad position e', bit dsh + 2 (g % 2).
  const uint32_t dsh = 8u * (uint32_t)(lane & 3) + 4u + (uint32_t)hh;
  const KeepConsts kq = keep_consts(p.drop.p8);
  uint32_t dc[4] = {0u, 0u, 0u, 0u};  // call in flight (the next chunk's)
  uint32_t dm = 0u;                   // ... packed
  uint32_t dM[2][4] = {};             // the current chunk's 8 calls, seen from this lane
  auto draw_init = [&](int row0) {    // first row of the chunk (a multiple of 32)
    dc[0] = (uint32_t)key >> 2;
    dc[1] = ((uint32_t)row0 >> 2) + 4u * (uint32_t)hh + (uint32_t)(lane & 3);
    dc[2] = (uint32_t)unit;
    dc[3] = 0u;
    dm = 0u;
  };
  // Item t of a call: rounds 0..9, then the keep bits of output word t - 10.
  auto draw_item = [&](int t) {
    if (t < 10) {
      philox_round(dc[0], dc[1], dc[2], dc[3], p.drop.seed_lo, p.drop.seed_hi, t);
    } else {
      dm = pack_keep(dm, keep_flags(dc[t - 10], kq), t - 10);  // row t - 10 of the block
    }
  };
  auto draw_share = [&]() {  // every lane's view of its 8-lane group's calls
    auto sw = __builtin_amdgcn_permlane32_swap(dm, dm, false, false);  // [0]: the half-0 lane's, [1]: the half-1 lane's
    dM[0][0] = quad_bcast<0>(sw[0]);
    dM[0][1] = quad_bcast<1>(sw[0]);
    dM[0][2] = quad_bcast<2>(sw[0]);
    dM[0][3] = quad_bcast<3>(sw[0]);
    dM[1][0] = quad_bcast<0>(sw[1]);
    dM[1][1] = quad_bcast<1>(sw[1]);
    dM[1][2] = quad_bcast<2>(sw[1]);
    dM[1][3] = quad_bcast<3>(sw[1]);
  };
  // Keep mask (all ones or zero) of register r of the current chunk.
  auto keep_mask = [&](int r) -> uint32_t {
    const int g = r >> 2, e = r & 3;
    return (uint32_t)__builtin_amdgcn_sbfe((int)dM[g >> 1][e], dsh + 2u * (uint32_t)(g & 1), 1u);
  };

  // One pipeline step for chunk (st, c): cur holds its S and dP (masked);
  // nxt receives S and dP of the next chunk (stage nst, chunk nc), computed
  // from whatever that stage holds (unused after the last chunk).
  //   phase A: MFMA S, dP (next chunk)   || VALU P, dS (this chunk)
  //   phase B: MFMA dV^T, dK^T (this chunk) with transposed reads
  // hook() runs in the third slice of the second phase (scalar set-up work).
  // lv holds this chunk's L log2(e) rows (f32x4 per row group); on return it
  // holds those of the next chunk.  dp arrives as dP - D (its accumulator
  // started from -D); dni is -D of the next chunk, the start of ndp.  With
  // dload, the second phase also reads -D of chunk 1 of stage nst into dnx.
  f32x4 lv[4];
  // Row operand i of a step's first phase (S, dP interleaved) for chunk c of stage st.
  auto arow = [&](int st, int c, int i) -> bf16x8 {
    const int si = (i * S::NQF) / S::NA, next = ((i + 1) * S::NQF) / S::NA;
    if (next > si) return *reinterpret_cast<const bf16x8*>(qs + st * S::QTILE + 32 * c * S::QS + qrb + 32 * si);
    return *reinterpret_cast<const bf16x8*>(os + st * S::OTILE + 32 * c * S::OS + orb + 32 * (i - si));
  };
  // First-phase row operands in flight across steps: a chunk-1 step loads the
  // first kPrefetchA operands of the following step (its stage is already
  // visible), which then starts without waiting for them.
  bf16x8 afr[kPrefetchA];
  // With DROP, dcur is -keep D of this chunk and nrow0 the first row of the next.
  auto step = [&](auto dofill, f32x16& sc, f32x16& dp, f32x16& nsc, f32x16& ndp, int st, int c, int nst, int nc,
                  const f32x16& dni, auto dload, f32x16& dnx, auto hook, auto pre_a, const f32x16& dcur, int nrow0) {
    const char* qb = qs + st * S::QTILE + 32 * c * S::QS + qtb;
    const char* ob = os + st * S::OTILE + 32 * c * S::OS + otb;
    const float* nls = reinterpret_cast<const float*>(lds_ld + nst * S::LDB + S::LD_L) + 32 * nc + 4 * hh;
    const float* nds = reinterpret_cast<const float*>(lds_ld + nst * S::LDB + S::LD_D) + 32 * 1 + 4 * hh;

    // MFMA j: even j -> dV block, odd -> dK block (while both remain).
    auto bmfma = [&](int j, bool& is_v, int& blk, int& ks) {
      constexpr int NV2 = 2 * S::NVB;
      const int vi = (j * NV2) / S::NB, vnext = ((j + 1) * NV2) / S::NB;
      is_v = vnext > vi;
      const int idx = is_v ? vi : j - vi;
      blk = idx % (is_v ? S::NVB : S::NDB);
      ks = idx / (is_v ? S::NVB : S::NDB);
    };
    auto bread = [&](int j, i16x4& lo, i16x4& hi) {
      bool is_v;
      int blk, ks;
      bmfma(j, is_v, blk, ks);
      const char* base = is_v ? ob : qb;
      const int stride = is_v ? S::OS : S::QS;
      lo = lds_read_tr(base + 16 * ks * stride, 64 * blk);
      hi = lds_read_tr(base + (16 * ks + 2) * stride, 64 * blk);
    };
    // ---- phase A ----
    constexpr int PF = kPrefetchA;  // row operands in flight
    auto aread = [&](int i) -> bf16x8 { return arow(nst, nc, i); };  // operand of MFMA i (S, dP interleaved)
    if constexpr (!decltype(pre_a)::value) {
#pragma unroll
      for (int i = 0; i < PF; ++i) afr[i] = aread(i);
    }
    // Transposed operands of the second phase: the first PB are read during
    // the first phase's last PB slices.
    constexpr int PB = kPrefetchB;
    i16x4 tlo[PB], thi[PB];
    u32x4 pk[2], sk[2];
    // Weights of row pair pr in two halves, issued one slice apart so that
    // the exponentials' latency is covered: e(pr) = exponentials, f(pr) = dS
    // and the bf16 packing.
    float pe[8][2];
    auto weights_e = [&](int pr) {
      const int r = 2 * pr, g = r >> 2, e = r & 3;
      pe[pr][0] = fast_exp2(__builtin_fmaf(sc[r], scale2, -lv[g][e]));
      pe[pr][1] = fast_exp2(__builtin_fmaf(sc[r + 1], scale2, -lv[g][e + 1]));
    };
    auto weights_f = [&](int pr) {
      const int r = 2 * pr;
      if constexpr (DROP) {  // dp = dP - keep D: keep dS = P (Z ? dp : -keep D)
        const uint32_t m0 = keep_mask(r), m1 = keep_mask(r + 1);
        const float z0 = __uint_as_float(__float_as_uint(pe[pr][0]) & m0);
        const float z1 = __uint_as_float(__float_as_uint(pe[pr][1]) & m1);
        const float v0 = __uint_as_float((__float_as_uint(dp[r]) & m0) | (__float_as_uint(dcur[r]) & ~m0));
        const float v1 = __uint_as_float((__float_as_uint(dp[r + 1]) & m1) | (__float_as_uint(dcur[r + 1]) & ~m1));
        const float d0 = pe[pr][0] * v0, d1 = pe[pr][1] * v1;
        pk[r >> 3][(r >> 1) & 3] = pack_bf16x2(z0, z1);
        sk[r >> 3][(r >> 1) & 3] = pack_bf16x2(d0, d1);
      } else {
        const float d0 = pe[pr][0] * dp[r];
        const float d1 = pe[pr][1] * dp[r + 1];
        pk[r >> 3][(r >> 1) & 3] = pack_bf16x2(pe[pr][0], pe[pr][1]);
        sk[r >> 3][(r >> 1) & 3] = pack_bf16x2(d0, d1);
      }
    };
    // Slices 0..8 over the NA MFMAs: slice k issues e(k) and f(k - 1).
#pragma unroll
    for (int i = 0; i < S::NA; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int si = (i * S::NQF) / S::NA, next = ((i + 1) * S::NQF) / S::NA;
      if (next > si) {
        if (si == 0) mfma_vz(nsc, afr[i % PF], kf[si]);
        else mfma_vacc(nsc, afr[i % PF], kf[si]);
      } else {
        if (i - si == 0) {
          mfma_vc(ndp, afr[i % PF], vf[i - si], dni);
        } else {
          mfma_vacc(ndp, afr[i % PF], vf[i - si]);
        }
      }
      if (i + PF < S::NA) afr[i % PF] = aread(i + PF);
      if (i >= S::NA - PB) bread(i - (S::NA - PB), tlo[i - (S::NA - PB)], thi[i - (S::NA - PB)]);
      if constexpr (decltype(dofill)::value) {
        if (i < FQ + FO) fill_item(i);
      }
#pragma unroll
      for (int k = i * 9 / S::NA; k < (i + 1) * 9 / S::NA; ++k) {
        if (k < 8) weights_e(k);
        if (k > 0) weights_f(k - 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"v"(dni));  // keep the init registers until its product is done

    // ---- phase B ----
    if constexpr (DROP) draw_init(nrow0);
    asm volatile("s_nop 1");  // the last packed P / dS operands were just written
    // Slice j: one MFMA, the reads PB MFMAs ahead and, for j < 8, one of the
    // next chunk's L log2(e) / D reads.
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      bool is_v;
      int blk, ks;
      bmfma(j, is_v, blk, ks);
      const bf16x8 a = join_tr(tlo[j % PB], thi[j % PB]);
      // (64, 64): the allocator moves accumulators through VGPRs (the
      // wait-state test of the compiled kernels checks every instance).
      constexpr bool kGuard = D == 64 && DV == 64;
      if (is_v) mfma_aacc_g<kGuard>(dv[blk], a, __builtin_bit_cast(bf16x8, pk[ks]));
      else mfma_aacc_g<kGuard>(dk[blk], a, __builtin_bit_cast(bf16x8, sk[ks]));
      if (j + PB < S::NB) bread(j + PB, tlo[j % PB], thi[j % PB]);
      if constexpr (decltype(dofill)::value) {  // chunk 1: the next step's first row operands
        if (j >= S::NB - PF) afr[j - (S::NB - PF)] = arow(nst, 1, j - (S::NB - PF));
      }
      if (j < 4) lv[j] = *reinterpret_cast<const f32x4*>(nls + 8 * j);
      if (j == 2) hook();
      if constexpr (DROP) {  // the next chunk's call: 14 items over the NB slices
#pragma unroll
        for (int t = j * 14 / S::NB; t < (j + 1) * 14 / S::NB; ++t) draw_item(t);
      }
      if constexpr (decltype(dload)::value) {
        if (j >= 4 && j < 8) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(nds + 8 * (j - 4));
#pragma unroll
          for (int e = 0; e < 4; ++e) dnx[4 * (j - 4) + e] = x[e];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DROP) draw_share();
  };

  // ---- main loop -------------------------------------------------------------
  int t0 = p.tq - 1;
  if (MASK == kMaskBitmask) {
    __syncthreads();  // tile classes staged
    if (t0 >= 0 && tile_class(t0) == kTileEmpty) t0 = next_tile(t0);
  }
  if (t0 < qt_first) t0 = -1;
  int t1 = next_tile(t0), t2 = next_tile(t1), t3 = next_tile(t2);
  int ntiles = 0;
  __syncthreads();  // ring cleared
  if (t0 >= 0) {  // workgroup-uniform
    fill(t0, 0);
    fill(t1, 1);
    fill(t2, 2);
    if constexpr (MASK != kMaskBitmask) plan_start(t2);
    wait_vm_n<2 * kF>();
    __syncthreads();
    f32x16 sa, pa, sb, pb;
    // -D of chunk 0 of the current tile (used by the dropout path's dS).
    f32x16 dnB = load_dn(0, 0);
    score_products(sa, pa, 0, 0, dnB);
    if constexpr (DROP) {  // the first chunk's calls
      draw_init(t0 * S::BQ);
#pragma unroll
      for (int t = 0; t < 14; ++t) draw_item(t);
      draw_share();
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      lv[g] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(lds_ld + S::LD_L) + 8 * g + 4 * hh);
    // -D starts of chunk 1 of the current tile (dnA) and chunk 0 of the next (dnB).
    f32x16 dnA = load_dn(0, 1);
#pragma unroll
    for (int i = 0; i < kPrefetchA; ++i) afr[i] = arow(0, 1, i);  // the first step's first operands
    unsigned j = 0;  // position of t0 in the sequence; its stage is j % NSTAGE
    while (true) {
      const int st = (int)(j & (S::NSTAGE - 1)), nst = (int)((j + 1) & (S::NSTAGE - 1));
      const int q0 = t0 * S::BQ;
      const bool partial = tile_partial(t0);
      // chunk 0 of t0
      if (partial) mask_chunk(sa, st, 0, q0);
      step(std::false_type{}, sa, pa, sb, pb, st, 0, st, 1, dnA, std::false_type{}, dnA,
           [&] { plan_fill(t3, (int)((j + 3) & (S::NSTAGE - 1))); }, std::true_type{}, dnB, q0 + 32);
      // The next tile's stage must be complete and visible before chunk 1's
      // phase A reads it; after this barrier every wave is past tile j-1, so
      // its stage takes the fill of position j+3.
      wait_vm_n<kF>();
      __syncthreads();
      dnB = load_dn(nst, 0);  // stage nst is complete after this barrier
      fill_begin();
      // chunk 1 of t0
      if (partial) mask_chunk(sb, st, 1, q0);
      step(std::true_type{}, sb, pb, sa, pa, st, 1, nst, 0, dnB, std::true_type{}, dnA, [] {}, std::false_type{}, dnA,
           t1 < 0 ? 0 : t1 * S::BQ);
      ++ntiles;
      if (t1 < 0) break;
      t0 = t1;
      t1 = t2;
      t2 = t3;
      t3 = next_tile(t2);
      ++j;
    }
    nops_after_mfma();  // the last dK^T / dV^T products were just issued
#pragma unroll
    for (int i = 0; i < S::NDB; ++i) after_nops_a(dk[i]);
#pragma unroll
    for (int i = 0; i < S::NVB; ++i) after_nops_a(dv[i]);
    wait_vm_n<0>();  // copies of empty positions
  }
  count_tiles(p.tile_count_kv, ntiles);

  // Epilogue: dK = c dK^T, dV = dV^T (lane = key; 4 consecutive columns per store).
  if (kvalid) {
    char* dKp = (char*)p.dK + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1] + (int64_t)key * p.sk[2]) * 2;
    char* dVp = (char*)p.dV + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1] + (int64_t)key * p.sv[2]) * 2;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = db * 32 + 8 * g + 4 * hh;
        const float sk = DROP ? p.scale * p.drop.keep_inv : p.scale;
        const float x0 = dk[db][4 * g] * sk, x1 = dk[db][4 * g + 1] * sk;
        const float x2 = dk[db][4 * g + 2] * sk, x3 = dk[db][4 * g + 3] * sk;
        *reinterpret_cast<u32x2*>(dKp + c0 * 2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      }
#pragma unroll
    for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = vb * 32 + 8 * g + 4 * hh;
        const float ks = DROP ? p.drop.keep_inv : 1.f;
        *reinterpret_cast<u32x2*>(dVp + c0 * 2) = u32x2{pack_bf16x2(dv[vb][4 * g] * ks, dv[vb][4 * g + 1] * ks),
                                                        pack_bf16x2(dv[vb][4 * g + 2] * ks, dv[vb][4 * g + 3] * ks)};
      }
  }
}

template <int D, int DV, int MASK>
static int launch_kv(const BwdParams& p, hipStream_t st) {
  if (p.drop.p8 != 0)
    hipLaunchKernelGGL((bwd_kv_kernel<D, DV, MASK, true>), dim3((unsigned)p.grid_pad), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<D, DV, MASK, false>), dim3((unsigned)p.grid_pad), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

template <int D, int DV>
static int launch_kv_mask(const BwdParams& p, int mask_mode, hipStream_t st) {
  switch (mask_mode) {
    case kMaskNone: return launch_kv<D, DV, kMaskNone>(p, st);
    case kMaskCausal: return launch_kv<D, DV, kMaskCausal>(p, st);
    default: return launch_kv<D, DV, kMaskBitmask>(p, st);
  }
}

bool bwd_kv_supported(int bf16, int d, int v, int mask_mode, int64_t tq) {
  if (!bf16 || !((d == 128 && v == 128) || (d == 64 && v == 128) || (d == 64 && v == 64))) return false;
  return mask_mode != kMaskBitmask || tq <= KvShape<128, 128>::MAXTQ;
}

int launch_bwd_kv(const BwdParams& p, int d, int v, int mask_mode, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (d == 128 && v == 128) return launch_kv_mask<128, 128>(p, mask_mode, st);
  if (d == 64 && v == 128) return launch_kv_mask<64, 128>(p, mask_mode, st);
  if (d == 64 && v == 64) return launch_kv_mask<64, 64>(p, mask_mode, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace eta
