// Backward, key-tile-outer dK / dV kernel at two waves per SIMD, for bf16
// with (d, v) = (128, 128), (64, 128) or (64, 64), no dropout and a none or
// causal mask: the main kernel of the deterministic backward in that case
// (dQ comes from the query-tile-outer kernel).
//
// Method (alphabetamath page, reverse procedure; ob1 page, part 2;
// HarshvardhanJ README, backward section): with the forward's L and
// D_i = <dO_i, O_i>, for each block recompute s_ij = c <Q_i, K_j>,
// p_ij = exp(s_ij - L_i), dP_ij = <dO_i, V_j>, dS_ij = p_ij (dP_ij - D_i), and
// accumulate dV_j += p_ij dO_i, dK_j += c dS_ij Q_i.  Query tiles that hold
// no allowed pair are skipped; only partially allowed tiles are masked (ob1
// page, part 3).
//
// gfx950 design.  One workgroup of eight waves per CU owns 256 keys, 32 per
// wave, so each SIMD runs two waves.  A wave keeps its K and V rows as MFMA B
// operands and its dK^T, dV^T accumulators in registers for the whole loop
// over query tiles (everything within 256 registers, VGPR-form MFMAs), and
// processes the two 32-row chunks of each 64-row query tile in turn: S = Q
// K^T and dP = dO V^T (dP starting from the stored -D, so that dS = P (dP -
// D) is one multiply) put one key in each lane column, so the registers
// holding P and dS are directly the B operand of dV^T += dO^T P and dK^T +=
// Q^T dS, whose dO^T / Q^T operands come from the row-major tiles through
// transposed LDS reads.  There is no software pipeline inside a wave: the
// other wave of the SIMD runs its MFMAs while this one waits for its scores
// or works on its weights.  The eight waves share one 4-stage ring of Q, dO,
// L log2(e) and -D tiles in LDS, filled straight from HBM (buffer_load ...
// lds from inline assembly, counted with vmcnt) three tiles ahead, with one
// barrier per tile; a tile copy serves 256 keys.  Tile rows are padded by 16
// bytes and the query rows of each group of 16 are taken in transposed order
// (4 u + v -> u + 4 v) by the score products, so the transposed reads of
// dO^T and Q^T cover rows 4 apart: both kinds of read are then free of bank
// conflicts.
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {

#ifndef ETA_KV2_PREFETCH_A
#define ETA_KV2_PREFETCH_A 2
#endif
#ifndef ETA_KV2_PREFETCH_C
#define ETA_KV2_PREFETCH_C 2
#endif
// Score-product read-ahead of the (128, 128) kernel without a mask: at depth
// 2 its register allocation spills a copy offset inside the main loop, and
// the reload's wait for all outstanding loads also waits for the tile copies
// just issued; at depth 1 nothing spills.
#ifndef ETA_KV2_PREFETCH_A_NOMASK
#define ETA_KV2_PREFETCH_A_NOMASK 1
#endif

template <int D, int DV>
struct Kv2Shape {
  static constexpr int NW = 8;
  static constexpr int BK = kBwdKv2Bk;  // keys per workgroup, 32 per wave
  static constexpr int BQ = kBwdBq;     // queries per tile: two chunks of 32
  static constexpr int NSTAGE = 4;      // LDS ring: tiles j .. j+3
  static constexpr int NQF = D / 16, NVF = DV / 16;  // K / V fragments per lane
  static constexpr int NDB = D / 32, NVB = DV / 32;  // 32-column blocks of dK^T / dV^T
  using QT = PadTile<D * 2, 16>;
  using OT = PadTile<DV * 2, 16>;
  static constexpr int QS = QT::kStride, OS = OT::kStride;
  static constexpr int QTILE = BQ * QS, OTILE = BQ * OS;
  static constexpr int QWINS = QTILE / 1024, OWINS = OTILE / 1024;  // 1 KB fill windows per tile
  static constexpr int QWIN = (QWINS + NW - 1) / NW, OWIN = (OWINS + NW - 1) / NW;
  // Per stage: -L log2(e) / (c log2(e)) [BQ], -D [BQ].
  static constexpr int LD_L = 0, LD_D = BQ * 4, LDB = 2 * BQ * 4;
  static_assert(QTILE % 1024 == 0 && OTILE % 1024 == 0, "whole fill windows");
  static_assert(BQ == 64 && BK == 32 * NW, "two chunks of 32 queries, 32 keys per wave");
};

template <int D, int DV, int MASK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_kv2_kernel(BwdParams p) {
  using S = Kv2Shape<D, DV>;
  static_assert(MASK != kMaskBitmask, "none and causal masks");
  __shared__ __attribute__((aligned(1024))) char qs[S::NSTAGE * S::QTILE];
  __shared__ __attribute__((aligned(1024))) char os[S::NSTAGE * S::OTILE];
  __shared__ __attribute__((aligned(16))) char lds_ld[S::NSTAGE * S::LDB];
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
  const int key = k0 + 32 * w + (lane & 31);
  const bool kvalid = key < nk;

  const int qrow = (int)p.sq[2] * 2, krow = (int)p.sk[2] * 2;
  const int vrow = (int)p.sv[2] * 2, orow = (int)p.so[2] * 2;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * 2;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * 2;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * 2;
  const char* dOb = (const char*)p.dO + ((int64_t)b * p.so[0] + (int64_t)h * p.so[1]) * 2;
  const float* Lsb = p.Ls + (int64_t)unit * p.n_pad;
  const float* Dnb = p.Dn + (int64_t)unit * p.n_pad;

  // Clear the ring once when the last query tile is partial: tile rows that a
  // fill leaves untouched (past n) then always hold finite values.
  if (n % S::BQ != 0) {
    for (int c = tid; c < S::NSTAGE * S::QTILE / 16; c += S::NW * kWave) reinterpret_cast<u32x4*>(qs)[c] = u32x4{0, 0, 0, 0};
    for (int c = tid; c < S::NSTAGE * S::OTILE / 16; c += S::NW * kWave) reinterpret_cast<u32x4*>(os)[c] = u32x4{0, 0, 0, 0};
    for (int c = tid; c < S::NSTAGE * S::LDB / 16; c += S::NW * kWave) reinterpret_cast<u32x4*>(lds_ld)[c] = u32x4{0, 0, 0, 0};
  }

  // Query-tile sequence: from the last tile down to the first that can hold
  // an allowed pair (causal: the tile containing row k0 - coff; past the last
  // row no query tile holds one).
  int qt_first = 0;
  if constexpr (MASK == kMaskCausal) {
    const int r0 = k0 - coff;
    qt_first = r0 >= n ? p.tq : (r0 > 0 ? r0 / S::BQ : 0);
  }
  // Partially allowed among the visited tiles: causal tiles from row t_full
  // on are full when every key of the workgroup exists.
  const bool keys_whole = k0 + S::BK <= nk;
  int t_full = 0;
  if constexpr (MASK == kMaskCausal) {
    const int r_full = k0 + S::BK - 1 - coff;  // first query row that allows every key of the tile
    t_full = r_full <= 0 ? 0 : (r_full + S::BQ - 1) / S::BQ;
  }
  auto tile_partial = [&](int qt) -> bool {
    if constexpr (MASK == kMaskCausal) return !(keys_whole && qt >= t_full);
    return !keys_whole;
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
    // Take the loads' completion here, where the compiler sees it: the tile
    // copies issued later in the loop are invisible to its wait counting,
    // so a wait it placed before a product in the loop would also wait for
    // the copies just issued.
#pragma unroll
    for (int s = 0; s < S::NQF; ++s) asm volatile("" : "+v"(kf[s]));
#pragma unroll
    for (int s = 0; s < S::NVF; ++s) asm volatile("" : "+v"(vf[s]));
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
  // Per tile every wave issues QWIN + OWIN tile copies and one row copy (the
  // score products' start -L log2(e) / (c log2(e)) by wave 0, -D by wave 1,
  // empty ranges by the others).
  constexpr int kF = S::QWIN + S::OWIN + 1;
  const i32x4 r_none = rsrc_words(Qb, 0);
  auto win_item = [&](const i32x4& r, uint32_t tile, int first, int nb, int nx, const auto& src, int i) {
    const bool extra = i == nb;
    const bool real = !extra || w < nx;
    if (i % 4 == 0 || extra)  // group start, or the item that may be an empty copy
      set_m0(real ? tile + (first + 4 * (i / 4)) * 1024 : sp_l);  // an empty copy lands at sp_l + (i % 4) KB
    // An empty copy keeps the resource's address and takes an empty range.
    fill16_off(i32x4{r[0], r[1], real ? r[2] : 0, r[3]}, src[i], i % 4);
  };
  // Buffer resource of the rows of query tile qt of a [n, row] slice with rb
  // bytes per row; the host bounds (n - 1) rb + the row width by 2^31 - 1, so
  // the products below fit in 32 bits.  qt < 0: an empty range.  Ranges are
  // clamped below 2^31: padding slots read at offset 2^31, which must stay out
  // of range.
  auto tile_words = [&](const void* base, int qt, int rb) -> i32x4 {
    const uint32_t q0 = qt < 0 ? 0u : (uint32_t)(qt * S::BQ);
    const uint32_t nb = qt < 0 ? 0u : (uint32_t)(n - (int)q0) * (uint32_t)rb;
    const uint64_t a = reinterpret_cast<uint64_t>(base) + q0 * (uint32_t)rb;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)(nb < 0x7FFFFFFFu ? nb : 0x7FFFFFFFu), 0x00020000};
  };
  // The copies of tile qt into stage st, item i of kF (qt < 0 copies nothing
  // but issues the same instructions).
  i32x4 frq, fro, frr;
  int fst = 0;
  auto plan = [&](int qt, int st) {
    frq = tile_words(Qb, qt, qrow);
    fro = tile_words(dOb, qt, orow);
    const float* src = (w == 0 ? Lsb : Dnb) + (qt < 0 ? 0 : qt * S::BQ);
    frr = (w < 2 && qt >= 0) ? rsrc_words(src, S::BQ * 4) : r_none;
    fst = st;
  };
  auto fill_item = [&](int i) {
    if (i < S::QWIN) {
      win_item(frq, qs_l + fst * S::QTILE, qfirst, QB, QX, qsrc, i);
    } else if (i < S::QWIN + S::OWIN) {
      win_item(fro, os_l + fst * S::OTILE, ofirst, OB, OX, osrc, i - S::QWIN);
    } else {  // padded rows: always in range; slot l holds row perm(l)
      fill4(frr, w < 2 ? ld_l + fst * S::LDB + (w == 0 ? S::LD_L : S::LD_D) : sp_l, 4 * perm(lane));
    }
  };

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

  // Exponent scale: c log2(e), with c = 0 replaced by 1e-30 (every finite
  // score then maps to exactly exp2(-L log2 e), as for c = 0, while the
  // masking sentinel below still maps to zero).
  const float scale2 = p.scale2 == 0.f ? 1e-30f : p.scale2;
  const float masked_score = scale2 > 0.f ? -INFINITY : INFINITY;  // exp2(score * scale2 - l) = 0

  // One 32-row chunk c of the tile in stage st (query rows q0 + 32 c ..), in
  // three phases whose instruction order is pinned by scheduling barriers:
  //   A: S and dP on the matrix cores (S and dP products interleaved, each
  //      operand read PA products ahead; with `copies`, one of the planned
  //      copies per product),
  //   W: P and dS on the vector ALUs, then the first transposed operands of C,
  //   C: dV^T and dK^T on the matrix cores (operands read PC products ahead).
  constexpr int NA = S::NQF + S::NVF;          // phase A products
  constexpr int NB = 2 * (S::NDB + S::NVB);    // phase C products
  constexpr int PA = (MASK == 0 && D == 128) ? ETA_KV2_PREFETCH_A_NOMASK : ETA_KV2_PREFETCH_A;  // operand reads in flight
  constexpr int PC = ETA_KV2_PREFETCH_C;
  auto chunk = [&](int st, int c, int q0, bool partial, bool copies) {
    const char* qb = qs + st * S::QTILE + 32 * c * S::QS;
    const char* ob = os + st * S::OTILE + 32 * c * S::OS;
    const float* ls = reinterpret_cast<const float*>(lds_ld + st * S::LDB + S::LD_L) + 32 * c + 4 * hh;
    const float* ds = reinterpret_cast<const float*>(lds_ld + st * S::LDB + S::LD_D) + 32 * c + 4 * hh;
    // Product i of phase A: S (fragment si) when the S share advances, else dP.
    auto a_is_s = [](int i) { return ((i + 1) * S::NQF) / NA > (i * S::NQF) / NA; };
    auto a_frag = [&](int i) { return a_is_s(i) ? (i * S::NQF) / NA : i - (i * S::NQF) / NA; };
    auto aread = [&](int i) -> bf16x8 {
      return a_is_s(i) ? *reinterpret_cast<const bf16x8*>(qb + qrb + 32 * a_frag(i))
                       : *reinterpret_cast<const bf16x8*>(ob + orb + 32 * a_frag(i));
    };
    // Product j of phase C: dV block (even j while both remain) or dK block.
    auto c_is_v = [](int j) { return ((j + 1) * 2 * S::NVB) / NB > (j * 2 * S::NVB) / NB; };
    auto c_idx = [&](int j) { return c_is_v(j) ? (j * 2 * S::NVB) / NB : j - (j * 2 * S::NVB) / NB; };
    i16x4 tlo[PC], thi[PC];
    auto bread = [&](int j) {
      const bool v = c_is_v(j);
      const int idx = c_idx(j), blk = idx % (v ? S::NVB : S::NDB), ks = idx / (v ? S::NVB : S::NDB);
      const char* base = v ? ob + otb + 16 * ks * S::OS : qb + qtb + 16 * ks * S::QS;
      const int stride = v ? S::OS : S::QS;
      tlo[j % PC] = lds_read_tr(base, 64 * blk);
      thi[j % PC] = lds_read_tr(base + 2 * stride, 64 * blk);
    };

    // S starts from -L log2(e) / (c log2(e)) and dP from -D: register r holds
    // row 8 (r / 4) + 4 hh + r % 4 of the chunk.  Then S c log2(e) is the
    // exponent s_ij log2(e) - L_i log2(e) of the weight.
    f32x16 sc, dp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(ls + 8 * j);
      const f32x4 y = *reinterpret_cast<const f32x4*>(ds + 8 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[4 * j + e] = x[e];
        dp[4 * j + e] = y[e];
      }
    }
    bf16x8 afr[PA];
#pragma unroll
    for (int i = 0; i < PA; ++i) afr[i] = aread(i);
    // ---- phase A ----
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 a = afr[i % PA];
      if (a_is_s(i)) {
        const int f = a_frag(i);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[f], sc, 0, 0, 0);
      } else {
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[a_frag(i)], dp, 0, 0, 0);
      }
      if (i + PA < NA) afr[i % PA] = aread(i + PA);
      if (copies && i < kF) fill_item(i);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (copies) {
#pragma unroll
      for (int i = NA; i < kF; ++i) fill_item(i);
    }
    // ---- phase W ----
    if (partial) {  // scores of disallowed pairs -> the sentinel
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * c + perm(8 * (r >> 2) + 4 * hh + (r & 3));
        bool ok = kvalid;
        if constexpr (MASK == kMaskCausal) ok = ok && key <= q0 + ql + coff;
        sc[r] = ok ? sc[r] : masked_score;
      }
    }
    // P = exp2(s c log2 e - L log2 e), dS = P (dP - D), packed as the B
    // operands of the gradient products (k index = chunk row).
    u32x4 pk[2], sk[2];
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      const int r = 2 * pr;
      const float p0 = fast_exp2(sc[r] * scale2);
      const float p1 = fast_exp2(sc[r + 1] * scale2);
      pk[r >> 3][(r >> 1) & 3] = pack_bf16x2(p0, p1);
      sk[r >> 3][(r >> 1) & 3] = pack_bf16x2(p0 * dp[r], p1 * dp[r + 1]);
    }
#pragma unroll
    for (int j = 0; j < PC; ++j) bread(j);
    // ---- phase C: dV^T += dO^T P and dK^T += Q^T dS over the chunk's rows ----
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      const bool v = c_is_v(j);
      const int idx = c_idx(j), blk = idx % (v ? S::NVB : S::NDB), ks = idx / (v ? S::NVB : S::NDB);
      const bf16x8 a = join_tr(tlo[j % PC], thi[j % PC]);
      if (v) dv[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pk[ks]), dv[blk], 0, 0, 0);
      else dk[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, sk[ks]), dk[blk], 0, 0, 0);
      if (j + PC < NB) bread(j + PC);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- main loop -------------------------------------------------------------
  // Tiles t0 > t1 > ... from the last query tile down to qt_first; tile j of
  // the sequence sits in stage j % 4.  Before tile j is processed its stage
  // is complete and visible, and the stage of tile j - 1 (free since the
  // barrier that ended tile j - 1) receives tile j + 3, whose copies are
  // issued during the first chunk's score products.
  int t0 = p.tq - 1;
  if (t0 < qt_first) t0 = -1;
  auto next = [&](int qt) { return qt - 1 >= qt_first ? qt - 1 : -1; };
  int t1 = t0 >= 0 ? next(t0) : -1, t2 = t1 >= 0 ? next(t1) : -1, t3 = t2 >= 0 ? next(t2) : -1;
  int ntiles = 0;
  __syncthreads();  // ring cleared
  if (t0 >= 0) {  // workgroup-uniform
    plan(t0, 0);
#pragma unroll
    for (int i = 0; i < kF; ++i) fill_item(i);
    plan(t1, 1);
#pragma unroll
    for (int i = 0; i < kF; ++i) fill_item(i);
    plan(t2, 2);
#pragma unroll
    for (int i = 0; i < kF; ++i) fill_item(i);
    wait_vm_n<0>();
    __syncthreads();
    unsigned j = 0;
    while (true) {
      const int st = (int)(j & (S::NSTAGE - 1));
      const int q0 = t0 * S::BQ;
      const bool partial = tile_partial(t0);
      plan(t3, (int)((j + 3) & (S::NSTAGE - 1)));
      chunk(st, 0, q0, partial, true);
      chunk(st, 1, q0, partial, false);
      ++ntiles;
      if (t1 < 0) break;
      // Tile j + 1 was copied two tiles ago; the copies of tiles j + 2 and
      // j + 3 may still be in flight.
      wait_vm_n<2 * kF>();
      __syncthreads();
      t0 = t1;
      t1 = t2;
      t2 = t3;
      t3 = t3 >= 0 ? next(t3) : -1;
      ++j;
    }
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
        const float x0 = dk[db][4 * g] * p.scale, x1 = dk[db][4 * g + 1] * p.scale;
        const float x2 = dk[db][4 * g + 2] * p.scale, x3 = dk[db][4 * g + 3] * p.scale;
        *reinterpret_cast<u32x2*>(dKp + c0 * 2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      }
#pragma unroll
    for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = vb * 32 + 8 * g + 4 * hh;
        *reinterpret_cast<u32x2*>(dVp + c0 * 2) = u32x2{pack_bf16x2(dv[vb][4 * g], dv[vb][4 * g + 1]),
                                                        pack_bf16x2(dv[vb][4 * g + 2], dv[vb][4 * g + 3])};
      }
  }
}

template <int D, int DV, int MASK>
static int launch_kv2(const BwdParams& p, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kv2_kernel<D, DV, MASK>), dim3((unsigned)p.grid_pad), dim3(Kv2Shape<D, DV>::NW * kWave),
                     0, st, p);
  return (int)hipGetLastError();
}

template <int D, int DV>
static int launch_kv2_mask(const BwdParams& p, int mask_mode, hipStream_t st) {
  if (mask_mode == kMaskCausal) return launch_kv2<D, DV, kMaskCausal>(p, st);
  return launch_kv2<D, DV, kMaskNone>(p, st);
}

int launch_bwd_kv2(const BwdParams& p, int d, int v, int mask_mode, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (mask_mode == kMaskBitmask) return (int)hipErrorInvalidValue;
  if (d == 128 && v == 128) return launch_kv2_mask<128, 128>(p, mask_mode, st);
  if (d == 64 && v == 128) return launch_kv2_mask<64, 128>(p, mask_mode, st);
  if (d == 64 && v == 64) return launch_kv2_mask<64, 64>(p, mask_mode, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace eta
