// Backward, key-tile-outer dK / dV kernel for bf16 with d, v in {64, 128}:
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
// wave keeps its K and V rows in registers as MFMA B operands and its dK^T,
// dV^T accumulators for the whole loop over query tiles.  Query tiles of 64
// rows are visited from the last one down and processed as two chunks of 32
// rows.  Per chunk, S = Q K^T and dP = dO V^T put one key in each lane
// column, so the registers holding P and dS are directly the B operand of
// dV^T += dO^T P and dK^T += Q^T dS, whose dO^T / Q^T operands come from the
// row-major tiles through transposed LDS reads.  The chunks form a software
// pipeline: the S / dP products of chunk k+1 run on the matrix cores while
// the vector ALUs turn chunk k's scores into P and dS, then chunk k's dV / dK
// products run; the instruction order is pinned with scheduling barriers.
// Q, dO, L log2(e) and D (and the bitmask words) are copied from HBM
// straight into a 4-stage ring of XOR-swizzled LDS tiles (buffer_load ...
// lds, issued from inline assembly and counted with vmcnt), two tiles ahead
// of their use, with one barrier per tile.  Every LDS read address is a
// per-lane register plus a constant.
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {


#ifndef ETA_KV_PREFETCH_A
#define ETA_KV_PREFETCH_A 4
#endif
#ifndef ETA_KV_PREFETCH_B
#define ETA_KV_PREFETCH_B 2
#endif
// LDS operand prefetch depth, in MFMAs, of the two phases.
constexpr int kPrefetchA = ETA_KV_PREFETCH_A, kPrefetchB = ETA_KV_PREFETCH_B;

template <int D, int DV>
struct KvShape {
  static constexpr int NW = 4;
  static constexpr int BK = kBwdBk;  // keys per workgroup, 32 per wave
  static constexpr int BQ = kBwdBq;  // queries per tile: two chunks of 32
  static constexpr int NSTAGE = 4;   // LDS ring: tiles j .. j+2 resident or in flight
  static constexpr int NQF = D / 16, NVF = DV / 16;  // K / V fragments per lane
  static constexpr int NDB = D / 32, NVB = DV / 32;  // 32-column blocks of dK^T / dV^T
  static constexpr int NA = NQF + NVF;               // S and dP MFMAs per chunk
  static constexpr int NB = 2 * (NDB + NVB);         // dK and dV MFMAs per chunk
  using QT = Swz<D / 8>;
  using OT = Swz<DV / 8>;
  static constexpr int QTILE = BQ * QT::kStride, OTILE = BQ * OT::kStride;
  static constexpr int QWIN = QTILE / 1024 / NW, OWIN = OTILE / 1024 / NW;  // 1 KB fills per wave
  static constexpr int MWORDS = BK / 32;
  // Per stage: L log2(e) [BQ], D [BQ], mask words [BQ][MWORDS].
  static constexpr int LD_L = 0, LD_D = BQ * 4, LD_M = 2 * BQ * 4;
  static constexpr int LDB = LD_M + BQ * MWORDS * 4;
  static constexpr int MAXTQ = 4096;  // bitmask: query tiles whose classes are staged in LDS
  static_assert(QT::kSwizzle && OT::kSwizzle && QT::kStride == D * 2 && OT::kStride == DV * 2, "layout");
  static_assert(QTILE % (1024 * NW) == 0 && OTILE % (1024 * NW) == 0, "tile fills");
  static_assert(BQ == 64 && BK == 128, "two chunks of 32 queries, 32 keys per wave");
};

template <int D, int DV, int MASK>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(BwdParams p) {
  using S = KvShape<D, DV>;
  __shared__ __attribute__((aligned(1024))) char qs[S::NSTAGE * S::QTILE];
  __shared__ __attribute__((aligned(1024))) char os[S::NSTAGE * S::OTILE];
  __shared__ __attribute__((aligned(16))) char lds_ld[S::NSTAGE * S::LDB];
  __shared__ uint8_t cls_s[MASK == kMaskBitmask ? S::MAXTQ : 1];

  const int64_t logical = xcd_logical(blockIdx.x, p.grid_pad, p.total);
  if (logical < 0) return;
  const int unit = (int)(logical / p.tk);
  const int kt = (int)(logical % p.tk);  // low key tiles (most causal work) first
  const int b = unit / p.H, h = unit % p.H;
  const int n = (int)p.n;
  const int k0 = kt * S::BK;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int g1 = (lane >> 4) & 1;
  const int klocal = 32 * w + (lane & 31);
  const int key = k0 + klocal;
  const bool kvalid = key < n;

  const int qrow = (int)p.sq[2] * 2, krow = (int)p.sk[2] * 2;
  const int vrow = (int)p.sv[2] * 2, orow = (int)p.so[2] * 2;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * 2;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * 2;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * 2;
  const char* dOb = (const char*)p.dO + ((int64_t)b * p.so[0] + (int64_t)h * p.so[1]) * 2;
  const float* L2b = p.L2 + (int64_t)unit * p.n_pad;
  const float* Db = p.Dv + (int64_t)unit * p.n_pad;
  const uint32_t* mbase = nullptr;
  if constexpr (MASK == kMaskBitmask) mbase = p.mask + b * p.mask_sb + h * p.mask_sh;

  // Clear the ring once: tile rows that a fill leaves untouched (past n)
  // then always hold finite values.
  for (int c = tid; c < S::NSTAGE * S::QTILE / 16; c += 256) reinterpret_cast<u32x4*>(qs)[c] = u32x4{0, 0, 0, 0};
  for (int c = tid; c < S::NSTAGE * S::OTILE / 16; c += 256) reinterpret_cast<u32x4*>(os)[c] = u32x4{0, 0, 0, 0};
  for (int c = tid; c < S::NSTAGE * S::LDB / 16; c += 256) reinterpret_cast<u32x4*>(lds_ld)[c] = u32x4{0, 0, 0, 0};

  // Query-tile sequence: from the last tile down to the first that can hold
  // an allowed pair (causal: the tile containing row k0); bitmask tiles come
  // from the tile map, staged in LDS so that the loop issues no loads of its own.
  int qt_first = 0;
  if constexpr (MASK == kMaskCausal) qt_first = k0 / S::BQ;
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    const uint8_t* map_col = p.map + mu * (int64_t)p.tq * p.tk + kt;
    for (int t = tid; t < p.tq; t += 256) cls_s[t] = map_col[(int64_t)t * p.tk];
  }
  auto tile_class = [&](int qt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return cls_s[qt];
    return classify_analytic(MASK, (int64_t)qt * S::BQ, S::BQ, k0, S::BK, n);
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
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb, n * krow);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vb, n * vrow);
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
  int qsrc[S::QWIN], osrc[S::OWIN];
#pragma unroll
  for (int i = 0; i < S::QWIN; ++i) qsrc[i] = S::QT::dma_src(w * S::QWIN + i, lane, qrow);
#pragma unroll
  for (int i = 0; i < S::OWIN; ++i) osrc[i] = S::OT::dma_src(w * S::OWIN + i, lane, orow);
  const uint32_t qs_l = lds_address(qs), os_l = lds_address(os), ld_l = lds_address(lds_ld);
  // Per tile, wave w issues QWIN + OWIN tile fills, waves 0 / 1 one more (L
  // log2(e) / D rows), and with a bitmask every wave one more (mask words of
  // 16 query rows).
  constexpr int kFillsA = S::QWIN + S::OWIN + 1 + (MASK == kMaskBitmask);  // waves 0, 1
  constexpr int kFillsB = S::QWIN + S::OWIN + (MASK == kMaskBitmask);      // waves 2, 3
  auto fill = [&](int qt, int st) {
    const int q0 = qt * S::BQ;
    const i32x4 rq = rsrc_words(Qb + (int64_t)q0 * qrow, (int64_t)(n - q0) * qrow);
    const i32x4 ro = rsrc_words(dOb + (int64_t)q0 * orow, (int64_t)(n - q0) * orow);
#pragma unroll
    for (int i = 0; i < S::QWIN; ++i) fill16(rq, qs_l + st * S::QTILE + (w * S::QWIN + i) * 1024, qsrc[i]);
#pragma unroll
    for (int i = 0; i < S::OWIN; ++i) fill16(ro, os_l + st * S::OTILE + (w * S::OWIN + i) * 1024, osrc[i]);
    if (w < 2) {  // padded rows: always in range
      const float* src = (w == 0 ? L2b : Db) + q0;
      fill4(rsrc_words(src, S::BQ * 4), ld_l + st * S::LDB + (w == 0 ? S::LD_L : S::LD_D), 4 * lane);
    }
    if constexpr (MASK == kMaskBitmask) {
      // Row 16 w + lane / 4 of the tile, word lane % 4 of this key tile.
      const int r = 16 * w + lane / 4;
      const i32x4 rm = rsrc_words(mbase + (int64_t)q0 * p.mask_si, (int64_t)(n - q0) * p.mask_si * 4);
      fill4(rm, ld_l + st * S::LDB + S::LD_M + 256 * w, (int)(((int64_t)r * p.mask_si + (k0 >> 5) + (lane & 3)) * 4));
    }
  };
  // Wait until at most k of this wave's tile fills are still in flight.
  auto wait_fills = [&](int k) {
    if (w < 2) {
      if (k <= 0) wait_vm_n<0>();
      else if (k == 1) wait_vm_n<kFillsA>();
      else wait_vm_n<2 * kFillsA>();
    } else {
      if (k <= 0) wait_vm_n<0>();
      else if (k == 1) wait_vm_n<kFillsB>();
      else wait_vm_n<2 * kFillsB>();
    }
  };

  // ---- per-lane LDS read addresses (stage and chunk offsets are constants) --
  // Row operands (S, dP): row lane % 32 of the chunk, chunk 2 ks + hh.
  int qra[S::NQF], ora[S::NVF];
#pragma unroll
  for (int s = 0; s < S::NQF; ++s) qra[s] = (int)S::QT::off(lane & 31, 2 * s + hh);
#pragma unroll
  for (int s = 0; s < S::NVF; ++s) ora[s] = (int)S::OT::off(lane & 31, 2 * s + hh);
  // Transposed operands (dK, dV): rows 4 hh + 8 half + i / 4, columns 32 blk + 16 g1.
  int qta[S::NDB][2], ota[S::NVB][2];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) qta[db][hf] = (int)S::QT::tr(lane, 8 * hf + 4 * hh, 32 * db + 16 * g1);
#pragma unroll
  for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) ota[vb][hf] = (int)S::OT::tr(lane, 8 * hf + 4 * hh, 32 * vb + 16 * g1);

  // S and dP of one chunk (32 query rows at tile row 32 c) from stage st.
  auto score_products = [&](f32x16& sc, f32x16& dp, int st, int c) {
    const char* qb = qs + st * S::QTILE + 32 * c * S::QT::kStride;
    const char* ob = os + st * S::OTILE + 32 * c * S::OT::kStride;
    sc = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int s = 0; s < S::NQF; ++s) sc = mfma_bf16(*reinterpret_cast<const bf16x8*>(qb + qra[s]), kf[s], sc);
#pragma unroll
    for (int s = 0; s < S::NVF; ++s) dp = mfma_bf16(*reinterpret_cast<const bf16x8*>(ob + ora[s]), vf[s], dp);
  };
  // Exponent scale: c log2(e), with c = 0 replaced by 1e-30 (every finite
  // score then maps to exactly exp2(-L log2 e), as for c = 0, while the
  // masking sentinel below still maps to zero).
  const float scale2 = p.scale2 == 0.f ? 1e-30f : p.scale2;
  const float masked_score = scale2 > 0.f ? -INFINITY : INFINITY;  // exp2(score * scale2 - l) = 0
  // Partially allowed tile: scores of disallowed pairs -> the sentinel.
  // Register r of a chunk holds query row 32 c + 8 (r / 4) + 4 hh + r % 4.
  auto mask_chunk = [&](f32x16& sc, int st, int c, int q0) {
    const uint32_t* ms = reinterpret_cast<const uint32_t*>(lds_ld + st * S::LDB + S::LD_M);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = 32 * c + 8 * (r >> 2) + 4 * hh + (r & 3);
      bool ok = kvalid;
      if constexpr (MASK == kMaskCausal) ok = ok && key <= q0 + ql;
      if constexpr (MASK == kMaskBitmask) ok = ok && ((ms[ql * S::MWORDS + w] >> (lane & 31)) & 1u);
      sc[r] = ok ? sc[r] : masked_score;
    }
  };

  // One pipeline step for chunk (st, c): cur holds its S and dP (masked);
  // nxt receives S and dP of the next chunk (stage nst, chunk nc), computed
  // from whatever that stage holds (unused after the last chunk).
  //   phase A: MFMA S, dP (next chunk)   || VALU P, dS (this chunk)
  //   phase B: MFMA dV^T, dK^T (this chunk) with transposed reads
  // lv / dvv hold this chunk's L log2(e) and D rows (f32x4 per row group);
  // on return they hold those of the next chunk.
  f32x4 lv[4], dvv[4];
  auto step = [&](f32x16& sc, f32x16& dp, f32x16& nsc, f32x16& ndp, int st, int c, int nst, int nc) {
    const char* nqb = qs + nst * S::QTILE + 32 * nc * S::QT::kStride;
    const char* nob = os + nst * S::OTILE + 32 * nc * S::OT::kStride;
    const char* qb = qs + st * S::QTILE + 32 * c * S::QT::kStride;
    const char* ob = os + st * S::OTILE + 32 * c * S::OT::kStride;
    const float* nls = reinterpret_cast<const float*>(lds_ld + nst * S::LDB + S::LD_L) + 32 * nc + 4 * hh;
    const float* nds = reinterpret_cast<const float*>(lds_ld + nst * S::LDB + S::LD_D) + 32 * nc + 4 * hh;

    // ---- phase A ----
    constexpr int PF = kPrefetchA;  // row operands in flight
    auto aread = [&](int i) -> bf16x8 {  // operand of MFMA i: dP (ks) or S (ks), interleaved
      const int si = (i * S::NQF) / S::NA, next = ((i + 1) * S::NQF) / S::NA;
      if (next > si) return *reinterpret_cast<const bf16x8*>(nqb + qra[si]);
      return *reinterpret_cast<const bf16x8*>(nob + ora[i - si]);
    };
    bf16x8 afr[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) afr[i] = aread(i);
    nsc = f32x16{};
    ndp = f32x16{};
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
      const int r = 2 * pr, g = r >> 2, e = r & 3;
      const float d0 = pe[pr][0] * (dp[r] - dvv[g][e]);
      const float d1 = pe[pr][1] * (dp[r + 1] - dvv[g][e + 1]);
      pk[r >> 3][(r >> 1) & 3] = pack_bf16x2(pe[pr][0], pe[pr][1]);
      sk[r >> 3][(r >> 1) & 3] = pack_bf16x2(d0, d1);
    };
    // Slices 0..8 over the NA MFMAs: slice k issues e(k) and f(k - 1).
#pragma unroll
    for (int i = 0; i < S::NA; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int si = (i * S::NQF) / S::NA, next = ((i + 1) * S::NQF) / S::NA;
      if (next > si) nsc = mfma_bf16(afr[i % PF], kf[si], nsc);
      else ndp = mfma_bf16(afr[i % PF], vf[i - si], ndp);
      if (i + PF < S::NA) afr[i % PF] = aread(i + PF);
#pragma unroll
      for (int k = i * 9 / S::NA; k < (i + 1) * 9 / S::NA; ++k) {
        if (k < 8) weights_e(k);
        if (k > 0) weights_f(k - 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase B ----
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
      const int stride = is_v ? S::OT::kStride : S::QT::kStride;
      const int a0 = is_v ? ota[blk][0] : qta[blk][0], a1 = is_v ? ota[blk][1] : qta[blk][1];
      lo = lds_read_tr(base + 16 * ks * stride, a0);
      hi = lds_read_tr(base + 16 * ks * stride, a1);
    };
    constexpr int PB = kPrefetchB;  // transposed operands in flight (MFMAs ahead)
    i16x4 tlo[PB], thi[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) bread(j, tlo[j], thi[j]);
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      bool is_v;
      int blk, ks;
      bmfma(j, is_v, blk, ks);
      const bf16x8 a = join_tr(tlo[j % PB], thi[j % PB]);
      if (is_v) dv[blk] = mfma_bf16(a, __builtin_bit_cast(bf16x8, pk[ks]), dv[blk]);
      else dk[blk] = mfma_bf16(a, __builtin_bit_cast(bf16x8, sk[ks]), dk[blk]);
      if (j + PB < S::NB) bread(j + PB, tlo[j % PB], thi[j % PB]);
      if (j == S::NB - 4) {  // next chunk's L log2(e) and D rows
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          lv[g] = *reinterpret_cast<const f32x4*>(nls + 8 * g);
          dvv[g] = *reinterpret_cast<const f32x4*>(nds + 8 * g);
        }
      }
    }
    // One MFMA, the reads PB MFMAs ahead, per group.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PB, 0);
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (j + PB < S::NB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      if (j == S::NB - 4) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- main loop -------------------------------------------------------------
  int t0 = p.tq - 1;
  if (MASK == kMaskBitmask) {
    __syncthreads();  // tile classes staged
    if (t0 >= 0 && tile_class(t0) == kTileEmpty) t0 = next_tile(t0);
  }
  if (t0 < qt_first) t0 = -1;
  int t1 = next_tile(t0), t2 = next_tile(t1), t3 = next_tile(t2);
  __syncthreads();  // ring cleared
  if (t0 >= 0) {  // workgroup-uniform
    int issued = 0;
    fill(t0, 0);
    ++issued;
    if (t1 >= 0) { fill(t1, 1); ++issued; }
    if (t2 >= 0) { fill(t2, 2); ++issued; }
    wait_fills(issued - 1);
    __syncthreads();
    f32x16 sa, pa, sb, pb;
    score_products(sa, pa, 0, 0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      lv[g] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(lds_ld + S::LD_L) + 8 * g + 4 * hh);
      dvv[g] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(lds_ld + S::LD_D) + 8 * g + 4 * hh);
    }
    int j = 0;  // position of t0 in the sequence; its stage is j % NSTAGE
    while (true) {
      const int st = j % S::NSTAGE, nst = (j + 1) % S::NSTAGE;
      const int q0 = t0 * S::BQ;
      const bool partial = tile_class(t0) == kTilePartial;
      // chunk 0 of t0
      if (partial) mask_chunk(sa, st, 0, q0);
      step(sa, pa, sb, pb, st, 0, st, 1);
      // The next tile's stage must be complete and visible before chunk 1's
      // phase A reads it; after this barrier every wave is past tile j-1, so
      // its stage takes the fill of position j+3.
      wait_fills(issued - (j + 2 < issued ? j + 2 : issued));
      __syncthreads();
      if (t3 >= 0) {
        fill(t3, (j + 3) % S::NSTAGE);
        ++issued;
      }
      // chunk 1 of t0
      if (partial) mask_chunk(sb, st, 1, q0);
      step(sb, pb, sa, pa, st, 1, nst, 0);
      if (t1 < 0) break;
      t0 = t1;
      t1 = t2;
      t2 = t3;
      t3 = next_tile(t2);
      ++j;
    }
  }

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
        *reinterpret_cast<u32x2*>(dVp + c0 * 2) =
            u32x2{pack_bf16x2(dv[vb][4 * g], dv[vb][4 * g + 1]), pack_bf16x2(dv[vb][4 * g + 2], dv[vb][4 * g + 3])};
      }
  }
}

template <int D, int DV, int MASK>
static int launch_kv(const BwdParams& p, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kv_kernel<D, DV, MASK>), dim3((unsigned)p.grid_pad), dim3(256), 0, st, p);
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
  if (!bf16 || !((d == 64 || d == 128) && (v == 64 || v == 128))) return false;
  return mask_mode != kMaskBitmask || tq <= KvShape<128, 128>::MAXTQ;
}

int launch_bwd_kv(const BwdParams& p, int d, int v, int mask_mode, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (d == 128 && v == 128) return launch_kv_mask<128, 128>(p, mask_mode, st);
  if (d == 64 && v == 128) return launch_kv_mask<64, 128>(p, mask_mode, st);
  if (d == 64 && v == 64) return launch_kv_mask<64, 64>(p, mask_mode, st);
  if (d == 128 && v == 64) return launch_kv_mask<128, 64>(p, mask_mode, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace eta
