// Backward, key-tile-outer kernel: dK, dV (and, fused, dQ by atomics).
//
// Method (alphabetamath page, reverse procedure; ob1 page, part 2;
// HarshvardhanJ README, backward section): with the forward's L and
// D_i = <dO_i, O_i>, for each block recompute s_ij = c <Q_i, K_j>,
// p_ij = exp(s_ij - L_i), dP_ij = <dO_i, V_j>, dS_ij = p_ij (dP_ij - D_i), and
// accumulate dV_j += p_ij dO_i, dK_j += c dS_ij Q_i (and dQ_i += c dS_ij K_j).
// No score or probability matrix is stored.
//
// gfx950 design.  One workgroup owns 128 keys (32 per wave); each wave keeps
// its K and V rows in registers as MFMA B operands and its dK^T, dV^T
// accumulators in registers for the whole loop over query tiles.  Per query
// tile the workgroup stages Q, dO, L and D through double-buffered,
// XOR-swizzled LDS (buffer loads: rows past n read as zero).  Scores and dP
// are formed as S = Q K^T and dP = dO V^T with one key per lane column, so
// the registers holding P and dS are directly the B operand of
// dV^T += dO^T P and dK^T += Q^T dS; the dO^T and Q^T operands come from the
// row-major LDS tiles through transposed reads whose addresses follow the
// order in which a lane holds its query rows.  Query tiles are visited from
// the last one down, so the workgroups of one head running together read
// the same Q and dO tiles.
//
// FUSED additionally forms dQ: dS is written to LDS (key-major) and read
// back with transposed reads as the A operand of dQ = dS K, added into an
// fp32 accumulator with buffer float atomics (rows past n are dropped by the
// buffer range check).  Without FUSED, dQ comes from the query-tile-outer
// kernel instead (deterministic, no atomics).
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {

template <bool BF16, int D, int DV>
struct BwdShape {
  static constexpr int NW = 4;
  static constexpr int BK = kBwdBk;             // keys per workgroup (32 per wave)
  static constexpr int BQ = BF16 ? kBwdBq : 32;  // queries per step
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int KSTEP = BF16 ? 16 : 2;
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int DVP = (DV + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  static constexpr int NVB = DVP / 32;
  static constexpr int NQB = BQ / 32;
  static constexpr int QCH = D * ES / 16;   // loaded chunks per Q row
  static constexpr int OCH = DV * ES / 16;  // loaded chunks per dO row
  using QT = Swz<DP * ES / 16>;
  using OT = Swz<DVP * ES / 16>;
  using KTl = Swz<DP * ES / 16>;  // resident K tile (fused dQ phase)
  using ST = Swz<BQ * ES / 16>;   // dS^T tile [key][query] (fused dQ phase)
  static constexpr int KTILE = BK * KTl::kStride;
  static constexpr int QTILE = BQ * QT::kStride;
  static constexpr int OTILE = BQ * OT::kStride;
  static constexpr int STILE = BK * ST::kStride;
  static constexpr int MWORDS = BK / 32;  // mask words per query row per key tile
  // Per buffer: Q tile, dO tile, L (base 2), D, mask words.
  static constexpr int BUF = QTILE + OTILE + BQ * 4 * 2 + BQ * MWORDS * 4;
  static constexpr int QLD = (BQ * QCH + 255) / 256;
  static constexpr int OLD = (BQ * OCH + 255) / 256;
  // Q and dO tiles go global -> LDS directly (buffer_load ... lds, 1 KiB of
  // lane-contiguous 16-byte chunks per wave instruction) when their rows are
  // unpadded and swizzled; each lane then fetches the logical chunk its
  // physical slot holds.
  static constexpr int QCPR = DP * ES / 16, OCPR = DVP * ES / 16;
  static constexpr bool DMA = BF16 && QT::kSwizzle && OT::kSwizzle && QCPR == QCH && OCPR == OCH &&
                              (BQ * QCPR) % (64 * NW) == 0 && (BQ * OCPR) % (64 * NW) == 0;
  static constexpr int QDMA = BQ * QCPR / (64 * NW), ODMA = BQ * OCPR / (64 * NW);  // per wave
  static constexpr int smem(bool fused) { return 2 * BUF + (fused ? KTILE + STILE : 0); }
};

// DROP: dropout replayed from the counter-based keep decisions of
// kern_common.h: dV^T += (P o Z)^T dO / keep, dS = P ((dO V^T) o Z / keep - D).
template <bool BF16, int D, int DV, int MASK, bool FUSED, bool DROP = false>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdParams p) {
  using S = BwdShape<BF16, D, DV>;
  __shared__ __attribute__((aligned(16))) char smem[S::smem(FUSED)];
  char* bufs = smem;
  char* Ks = smem + 2 * S::BUF;     // fused only
  char* dSs = Ks + S::KTILE;        // fused only

  const int64_t logical = xcd_logical(blockIdx.x, p.grid_pad, p.total);
  if (logical < 0) return;
  const int unit = (int)(logical / p.tk);
  const int kt = (int)(logical % p.tk);  // low key tiles (most causal work) first
  const int b = unit / p.H, h = unit % p.H;
  const int n = (int)p.n, nk = (int)p.nk, coff = (int)p.coff;  // query rows, key rows, causal offset
  const int k0 = kt * S::BK;

  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int hh = lane >> 5;
  const int g1 = (lane >> 4) & 1;
  const int klocal = 32 * w + (lane & 31);
  const int key = k0 + klocal;
  const bool kvalid = key < nk;

  const int qrow = (int)p.sq[2] * S::ES, krow = (int)p.sk[2] * S::ES;
  const int vrow = (int)p.sv[2] * S::ES, orow = (int)p.so[2] * S::ES;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * S::ES;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * S::ES;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * S::ES;
  const char* dOb = (const char*)p.dO + ((int64_t)b * p.so[0] + (int64_t)h * p.so[1]) * S::ES;
  const float* Lb = p.L + (int64_t)unit * n;
  const float* Dnb = p.Dn + (int64_t)unit * p.n_pad;

  if constexpr (FUSED) {
    // Resident K tile in LDS (B operand of dQ), padded columns cleared.
    constexpr int KCH = S::DP * S::ES / 16;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb + (int64_t)k0 * krow, (int64_t)(nk - k0) * krow);
    for (int c = tid; c < S::BK * KCH; c += 256) {
      const int r = c / KCH, cc = c % KCH;
      u32x4 x = u32x4{0, 0, 0, 0};
      if (cc * 16 < D * S::ES) x = __builtin_amdgcn_raw_buffer_load_b128(rk, r * krow + cc * 16, 0, 0);
      *reinterpret_cast<u32x4*>(Ks + S::KTl::off(r, cc)) = x;
    }
  }
  // Direct-to-LDS staging: start from zeroed buffers, so rows the range
  // check drops never hold stale non-finite patterns.
  if constexpr (S::DMA) {
    for (int c = tid; c < 2 * S::BUF / 16; c += 256) reinterpret_cast<u32x4*>(bufs)[c] = u32x4{0, 0, 0, 0};
    __syncthreads();  // cleared before any wave's direct loads land
  }
  // Clear the padded columns of both Q / dO buffers once.
  if constexpr (S::DP != D || S::DVP != DV) {
    for (int bi = 0; bi < 2; ++bi) {
      char* Qs = bufs + bi * S::BUF;
      char* Os = Qs + S::QTILE;
      constexpr int qpc = (S::DP - D) * S::ES / 16, opc = (S::DVP - DV) * S::ES / 16;
      for (int c = tid; c < S::BQ * qpc; c += 256)
        *reinterpret_cast<u32x4*>(Qs + S::QT::off(c / qpc, S::QCH + c % qpc)) = u32x4{0, 0, 0, 0};
      for (int c = tid; c < S::BQ * opc; c += 256)
        *reinterpret_cast<u32x4*>(Os + S::OT::off(c / opc, S::OCH + c % opc)) = u32x4{0, 0, 0, 0};
    }
  }

  // Per-wave K and V rows as B operands (lane column = its key).
  typedef typename std::conditional<BF16, bf16x8, float>::type Frag;
  constexpr int NKF = D / S::KSTEP, NVF = DV / S::KSTEP;
  Frag kf[NKF], vf[NVF];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb, (int64_t)nk * krow);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vb, (int64_t)nk * vrow);
#pragma unroll
    for (int s = 0; s < NKF; ++s) {
      if constexpr (BF16)
        kf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, key * krow + (16 * s + 8 * hh) * 2, 0, 0));
      else
        kf[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rk, key * krow + (2 * s + hh) * 4, 0, 0));
    }
#pragma unroll
    for (int s = 0; s < NVF; ++s) {
      if constexpr (BF16)
        vf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, key * vrow + (16 * s + 8 * hh) * 2, 0, 0));
      else
        vf[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, key * vrow + (2 * s + hh) * 4, 0, 0));
    }
  }

  f32x16 dk[S::NDB], dv[S::NVB];
#pragma unroll
  for (int i = 0; i < S::NDB; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < S::NVB; ++i) dv[i] = f32x16{};

  // Query tiles are visited from the last down to the first one that can
  // hold an allowed pair (causal: the tile containing row k0 - coff).
  int qt_first = 0;
  if constexpr (MASK == kMaskCausal) {
    // Row k0 - coff is the first that allows key k0.  Past the last row no
    // query tile holds an allowed pair: the tile containing that padding row
    // is empty, not partial, and must not be visited.
    const int r0 = k0 - coff;
    qt_first = r0 >= n ? p.tq : (r0 > 0 ? r0 / S::BQ : 0);
  }
  const uint8_t* map_col = nullptr;
  const uint32_t* mbase = nullptr;
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    map_col = p.map + mu * (int64_t)p.tq * p.tk + kt;
    mbase = p.mask + b * p.mask_sb + h * p.mask_sh;
  }
  auto tile_class = [&](int qt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return map_col[(int64_t)qt * p.tk];
    return classify_analytic(MASK, (int64_t)qt * S::BQ, S::BQ, k0, S::BK, n, nk, coff);
  };
  auto next_tile = [&](int qt) -> int {  // next (lower) tile with an allowed pair, or -1
    if constexpr (MASK != kMaskBitmask) return qt - 1 >= qt_first ? qt - 1 : -1;
    for (int t = qt - 1; t >= qt_first; --t)
      if (tile_class(t) != kTileEmpty) return t;
    return -1;
  };

  u32x4 qreg[S::QLD], oreg[S::OLD];
  float lreg = 0.f, dreg = 0.f;
  uint32_t mreg = 0;
  auto gload = [&](int qt, int bi) {
    const int q0 = qt * S::BQ;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb + (int64_t)q0 * qrow, (int64_t)(n - q0) * qrow);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(dOb + (int64_t)q0 * orow, (int64_t)(n - q0) * orow);
    if constexpr (S::DMA) {
      char* Qs = bufs + bi * S::BUF;
      char* Os = Qs + S::QTILE;
#pragma unroll
      for (int j = 0; j < S::QDMA; ++j) {
        const int inst = w * S::QDMA + j, idx = inst * 64 + lane;
        const int r = idx / S::QCPR, c = S::QT::chunk(r, idx % S::QCPR);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(Qs + inst * 1024), 16,
                                                 r * qrow + c * 16, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < S::ODMA; ++j) {
        const int inst = w * S::ODMA + j, idx = inst * 64 + lane;
        const int r = idx / S::OCPR, c = S::OT::chunk(r, idx % S::OCPR);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (__attribute__((address_space(3))) void*)(Os + inst * 1024), 16,
                                                 r * orow + c * 16, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < S::QLD * !S::DMA; ++i) {
      const int c = tid + i * 256;
      if (S::BQ * S::QCH % 256 == 0 || c < S::BQ * S::QCH)
        qreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, (c / S::QCH) * qrow + (c % S::QCH) * 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < S::OLD * !S::DMA; ++i) {
      const int c = tid + i * 256;
      if (S::BQ * S::OCH % 256 == 0 || c < S::BQ * S::OCH)
        oreg[i] = __builtin_amdgcn_raw_buffer_load_b128(ro, (c / S::OCH) * orow + (c % S::OCH) * 16, 0, 0);
    }
    if (tid < S::BQ) {
      const int qq = q0 + tid;
      const float Lv = qq < n ? Lb[qq] : -INFINITY;
      // Rows with L = -inf (no allowed key, or past n) get +inf: p = exp2(s - inf) = 0.
      lreg = (Lv == -INFINITY) ? INFINITY : Lv * kLog2e;
      dreg = qq < n ? -Dnb[qq] : 0.f;
    }
    if constexpr (MASK == kMaskBitmask) {
      if (tid < S::BQ * S::MWORDS) {
        const int r = tid / S::MWORDS, wi = tid % S::MWORDS;
        const int qq = q0 + r;
        const int wd = (k0 >> 5) + wi;
        mreg = (qq < n && wd * 32 < nk) ? mbase[(int64_t)qq * p.mask_si + wd] : 0u;
      }
    }
  };
  auto lstore = [&](int bi) {
    char* Qs = bufs + bi * S::BUF;
    char* Os = Qs + S::QTILE;
    float* Ls = reinterpret_cast<float*>(Os + S::OTILE);
    float* Dsv = Ls + S::BQ;
    uint32_t* Ms = reinterpret_cast<uint32_t*>(Dsv + S::BQ);
#pragma unroll
    for (int i = 0; i < S::QLD * !S::DMA; ++i) {
      const int c = tid + i * 256;
      if (S::BQ * S::QCH % 256 == 0 || c < S::BQ * S::QCH)
        *reinterpret_cast<u32x4*>(Qs + S::QT::off(c / S::QCH, c % S::QCH)) = qreg[i];
    }
#pragma unroll
    for (int i = 0; i < S::OLD * !S::DMA; ++i) {
      const int c = tid + i * 256;
      if (S::BQ * S::OCH % 256 == 0 || c < S::BQ * S::OCH)
        *reinterpret_cast<u32x4*>(Os + S::OT::off(c / S::OCH, c % S::OCH)) = oreg[i];
    }
    if (tid < S::BQ) {
      Ls[tid] = lreg;
      Dsv[tid] = dreg;
    }
    if constexpr (MASK == kMaskBitmask) {
      if (tid < S::BQ * S::MWORDS) Ms[tid] = mreg;
    }
  };

  __amdgpu_buffer_rsrc_t rdq;  // fused: dQ accumulator rows of this unit
  if constexpr (FUSED) rdq = make_rsrc(p.dQacc + (int64_t)unit * n * D, (int64_t)n * D * 4);

  int qt = p.tq - 1;
  if (MASK == kMaskBitmask && qt >= qt_first && tile_class(qt) == kTileEmpty) qt = next_tile(qt);
  if (qt < qt_first) qt = -1;
  if (qt >= 0) {
    gload(qt, 0);
    lstore(0);
  }
  if constexpr (S::DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's direct loads landed
  __syncthreads();
  int buf = 0, ntiles = 0;

  while (qt >= 0) {
    const int nq = next_tile(qt);
    const uint8_t cls = tile_class(qt);
    if (nq >= 0) gload(nq, buf ^ 1);
    const int q0 = qt * S::BQ;
    const char* Qs = bufs + buf * S::BUF;
    const char* Os = Qs + S::QTILE;
    const float* Ls = reinterpret_cast<const float*>(Os + S::OTILE);
    const float* Dsv = Ls + S::BQ;
    const uint32_t* Ms = reinterpret_cast<const uint32_t*>(Dsv + S::BQ);

    bool active = true;
    if constexpr (MASK == kMaskCausal) active = (k0 + 32 * w) <= (q0 + S::BQ - 1 + coff);  // wave-uniform
    if (active) {
#pragma unroll
      for (int qb = 0; qb < S::NQB; ++qb) {
        // S = Q K^T and dP = dO V^T for 32 query rows x this wave's 32 keys.
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < NKF; ++s) {
          if constexpr (BF16)
            sc = mfma_bf16(lds_read_b128(Qs, S::QT::off(32 * qb + (lane & 31), 2 * s + hh)), kf[s], sc);
          else
            sc = mfma_f32(*reinterpret_cast<const float*>(Qs + S::QT::off_dword(32 * qb + (lane & 31), 2 * s + hh)),
                          kf[s], sc);
        }
#pragma unroll
        for (int s = 0; s < NVF; ++s) {
          if constexpr (BF16)
            dp = mfma_bf16(lds_read_b128(Os, S::OT::off(32 * qb + (lane & 31), 2 * s + hh)), vf[s], dp);
          else
            dp = mfma_f32(*reinterpret_cast<const float*>(Os + S::OT::off_dword(32 * qb + (lane & 31), 2 * s + hh)),
                          vf[s], dp);
        }
        // P = exp2(s c log2e - L log2e); dS = P (dP - D).  Register r holds
        // query row 32 qb + 8 (r/4) + 4 hh + r%4 of the tile.
        // Dropout: rows 4g'..4g'+3 (g' = 8 g + 4 hh in the tile) of this lane's
        // key form one draw group; the quad's lanes hold keys 4a..4a+3, so lane
        // e of the quad draws group e for all four keys (keep_mask16) and each
        // lane takes its key's nibble of every group.
        uint32_t keepg[4] = {0xFu, 0xFu, 0xFu, 0xFu};
        if constexpr (DROP) {
          const uint32_t e = (uint32_t)lane & 3u;
          const uint32_t m = keep_mask16(p.drop.seed_lo, p.drop.seed_hi, p.drop.p8, (uint32_t)key >> 2,
                                         (uint32_t)(q0 + 32 * qb + 8 * (int)e + 4 * hh) >> 2, (uint32_t)unit, true);
          keepg[0] = (quad_bcast<0>(m) >> (4 * e)) & 0xFu;
          keepg[1] = (quad_bcast<1>(m) >> (4 * e)) & 0xFu;
          keepg[2] = (quad_bcast<2>(m) >> (4 * e)) & 0xFu;
          keepg[3] = (quad_bcast<3>(m) >> (4 * e)) & 0xFu;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = 32 * qb + 8 * g + 4 * hh;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + ql);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dsv + ql);
          const uint32_t keep = keepg[g];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pv = fast_exp2(__builtin_fmaf(sc[r], p.scale2, -l4[e]));
            if (cls == kTilePartial) {
              const int qq = q0 + ql + e;
              bool ok = kvalid;
              if constexpr (MASK == kMaskCausal) ok = ok && key <= qq + coff;
              if constexpr (MASK == kMaskBitmask)
                ok = ok & (((Ms[(ql + e) * S::MWORDS + (klocal >> 5)] >> (klocal & 31)) & 1u) != 0u);  // no short-circuit: no branch per read
              pv = ok ? pv : 0.f;
            }
            if constexpr (DROP) {
              const bool z = (keep >> e) & 1u;
              sc[r] = z ? pv : 0.f;
              dp[r] = pv * ((z ? dp[r] : 0.f) - d4[e]) * p.drop.keep_inv;  // d4 = D P(keep)
            } else {
              sc[r] = pv;
              dp[r] = pv * (dp[r] - d4[e]);
            }
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS.
        if constexpr (BF16) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const u32x4 pw{pack_bf16x2(sc[8 * ks], sc[8 * ks + 1]), pack_bf16x2(sc[8 * ks + 2], sc[8 * ks + 3]),
                           pack_bf16x2(sc[8 * ks + 4], sc[8 * ks + 5]), pack_bf16x2(sc[8 * ks + 6], sc[8 * ks + 7])};
            const u32x4 sw{pack_bf16x2(dp[8 * ks], dp[8 * ks + 1]), pack_bf16x2(dp[8 * ks + 2], dp[8 * ks + 3]),
                           pack_bf16x2(dp[8 * ks + 4], dp[8 * ks + 5]), pack_bf16x2(dp[8 * ks + 6], dp[8 * ks + 7])};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
            const bf16x8 sb = __builtin_bit_cast(bf16x8, sw);
            const int kr = 32 * qb + 16 * ks + 4 * hh;
#pragma unroll
            for (int vb = 0; vb < S::NVB; ++vb) {
              const int n0 = vb * 32 + 16 * g1;
              const i16x4 lo = lds_read_tr(Os, S::OT::tr(lane, kr, n0));
              const i16x4 hi = lds_read_tr(Os, S::OT::tr(lane, kr + 8, n0));
              dv[vb] = mfma_bf16(join_tr(lo, hi), pb, dv[vb]);
            }
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              const int n0 = db * 32 + 16 * g1;
              const i16x4 lo = lds_read_tr(Qs, S::QT::tr(lane, kr, n0));
              const i16x4 hi = lds_read_tr(Qs, S::QT::tr(lane, kr + 8, n0));
              dk[db] = mfma_bf16(join_tr(lo, hi), sb, dk[db]);
            }
            if constexpr (FUSED) {
              // dS^T -> LDS (key-major): 4 consecutive query rows per 8-byte store.
#pragma unroll
              for (int gg = 0; gg < 2; ++gg) {
                const int g = 2 * ks + gg;
                const int ql = 32 * qb + 8 * g + 4 * hh;
                *reinterpret_cast<u32x2*>(dSs + S::ST::off(klocal, ql >> 3) + 8 * ((ql >> 2) & 1)) =
                    u32x2{sw[2 * gg], sw[2 * gg + 1]};
              }
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
            for (int vb = 0; vb < S::NVB; ++vb) {
              const float a = *reinterpret_cast<const float*>(Os + S::OT::off_dword(ql, vb * 32 + (lane & 31)));
              dv[vb] = mfma_f32(a, sc[r], dv[vb]);
            }
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              const float a = *reinterpret_cast<const float*>(Qs + S::QT::off_dword(ql, db * 32 + (lane & 31)));
              dk[db] = mfma_f32(a, dp[r], dk[db]);
            }
          }
          if constexpr (FUSED) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int ql = 32 * qb + 8 * g + 4 * hh;
              *reinterpret_cast<f32x4*>(dSs + S::ST::off(klocal, ql >> 2)) =
                  f32x4{dp[4 * g], dp[4 * g + 1], dp[4 * g + 2], dp[4 * g + 3]};
            }
          }
        }
      }
    } else if constexpr (FUSED) {
      // All of this wave's keys are masked for the tile: its dS rows are zero.
      for (int c = lane; c < 32 * S::BQ * S::ES / 16; c += kWave) {
        const int r = c / (S::BQ * S::ES / 16), cc = c % (S::BQ * S::ES / 16);
        *reinterpret_cast<u32x4*>(dSs + S::ST::off(32 * w + r, cc)) = u32x4{0, 0, 0, 0};
      }
    }

    if constexpr (FUSED) {
      __syncthreads();  // dS of all 128 keys in LDS
      // dQ (this query tile, all d) += dS K over the workgroup's 128 keys.
      for (int blk = w; blk < S::NQB * S::NDB; blk += S::NW) {
        const int qb = blk % S::NQB, db = blk / S::NQB;
        f32x16 acc = f32x16{};
        if constexpr (BF16) {
#pragma unroll
          for (int ks = 0; ks < S::BK / 16; ++ks) {
            const int kr = 16 * ks + 8 * hh;
            const i16x4 alo = lds_read_tr(dSs, S::ST::tr(lane, kr, 32 * qb + 16 * g1));
            const i16x4 ahi = lds_read_tr(dSs, S::ST::tr(lane, kr + 4, 32 * qb + 16 * g1));
            const i16x4 blo = lds_read_tr(Ks, S::KTl::tr(lane, kr, 32 * db + 16 * g1));
            const i16x4 bhi = lds_read_tr(Ks, S::KTl::tr(lane, kr + 4, 32 * db + 16 * g1));
            acc = mfma_bf16(join_tr(alo, ahi), join_tr(blo, bhi), acc);
          }
        } else {
#pragma unroll 8
          for (int ks = 0; ks < S::BK / 2; ++ks) {
            const int kr = 2 * ks + hh;
            const float a = *reinterpret_cast<const float*>(dSs + S::ST::off_dword(kr, 32 * qb + (lane & 31)));
            const float bb = *reinterpret_cast<const float*>(Ks + S::KTl::off_dword(kr, 32 * db + (lane & 31)));
            acc = mfma_f32(a, bb, acc);
          }
        }
        const int dcol = 32 * db + (lane & 31);
        if (dcol < D) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qq = q0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], rdq, (qq * D + dcol) * 4, 0, 0);
          }
        }
      }
    }

    if (nq >= 0) lstore(buf ^ 1);
    if constexpr (S::DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf ^= 1;
    qt = nq;
    ++ntiles;
  }
  count_tiles(p.tile_count_kv, ntiles);

  // Epilogue: dK = c dK^T, dV = dV^T (lane = key; 4 consecutive columns per store).
  if (kvalid) {
    char* dKp = (char*)p.dK + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1] + (int64_t)key * p.sk[2]) * S::ES;
    char* dVp = (char*)p.dV + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1] + (int64_t)key * p.sv[2]) * S::ES;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = db * 32 + 8 * g + 4 * hh;
        if (c0 < D) {
          const float x0 = dk[db][4 * g] * p.scale, x1 = dk[db][4 * g + 1] * p.scale;
          const float x2 = dk[db][4 * g + 2] * p.scale, x3 = dk[db][4 * g + 3] * p.scale;
          if constexpr (BF16)
            *reinterpret_cast<u32x2*>(dKp + c0 * 2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          else
            *reinterpret_cast<f32x4*>(dKp + c0 * 4) = f32x4{x0, x1, x2, x3};
        }
      }
#pragma unroll
    for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = vb * 32 + 8 * g + 4 * hh;
        if (c0 < DV) {
          const float ks = DROP ? p.drop.keep_inv : 1.f;
          const float x0 = dv[vb][4 * g] * ks, x1 = dv[vb][4 * g + 1] * ks;
          const float x2 = dv[vb][4 * g + 2] * ks, x3 = dv[vb][4 * g + 3] * ks;
          if constexpr (BF16)
            *reinterpret_cast<u32x2*>(dVp + c0 * 2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          else
            *reinterpret_cast<f32x4*>(dVp + c0 * 4) = f32x4{x0, x1, x2, x3};
        }
      }
  }
}

template <bool BF16, int D, int DV, int MASK>
static int launch_one(const BwdParams& p, bool fused, hipStream_t st) {
  const dim3 grid((unsigned)p.grid_pad), block(256);
  if (p.drop.p8 != 0) {
    if (fused) hipLaunchKernelGGL((bwd_kernel<BF16, D, DV, MASK, true, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((bwd_kernel<BF16, D, DV, MASK, false, true>), grid, block, 0, st, p);
  } else if (fused) {
    hipLaunchKernelGGL((bwd_kernel<BF16, D, DV, MASK, true>), grid, block, 0, st, p);
  } else {
    hipLaunchKernelGGL((bwd_kernel<BF16, D, DV, MASK, false>), grid, block, 0, st, p);
  }
  return (int)hipGetLastError();
}

template <bool BF16, int D, int DV>
static int launch_mask(const BwdParams& p, int mask_mode, bool fused, hipStream_t st) {
  switch (mask_mode) {
    case kMaskNone: return launch_one<BF16, D, DV, kMaskNone>(p, fused, st);
    case kMaskCausal: return launch_one<BF16, D, DV, kMaskCausal>(p, fused, st);
    default: return launch_one<BF16, D, DV, kMaskBitmask>(p, fused, st);
  }
}

template <bool BF16>
static int launch_dims(const BwdParams& p, int d, int v, int mask_mode, bool fused, hipStream_t st) {
  if (d == 64 && v == 64) return launch_mask<BF16, 64, 64>(p, mask_mode, fused, st);
  if (d == 80 && v == 80) return launch_mask<BF16, 80, 80>(p, mask_mode, fused, st);
  if (d == 128 && v == 128) return launch_mask<BF16, 128, 128>(p, mask_mode, fused, st);
  if (d == 64 && v == 128) return launch_mask<BF16, 64, 128>(p, mask_mode, fused, st);
  return (int)hipErrorInvalidValue;
}

int launch_bwd(const BwdParams& p, int bf16, int d, int v, int mask_mode, bool fused, void* stream) {
  if (bwd_kv2_supported(bf16, d, v, mask_mode, fused, p.drop.p8)) return launch_bwd_kv2(p, d, v, mask_mode, stream);
  if (!fused && bwd_kv_supported(bf16, d, v, mask_mode, p.tq))
    return launch_bwd_kv(p, d, v, mask_mode, stream);
  hipStream_t st = (hipStream_t)stream;
  return bf16 ? launch_dims<true>(p, d, v, mask_mode, fused, st)
              : launch_dims<false>(p, d, v, mask_mode, fused, st);
}

}  // namespace eta
