// Backward kernel: block-recomputed vector-Jacobian product.
//
// Method (alphabetamath page, reverse procedure; ob1 page, part 2;
// HarshvardhanJ README, backward section): with the forward's L and
// D_i = <dO_i, O_i>, for each block recompute s_ij = c <Q_i, K_j>,
// p_ij = exp(s_ij - L_i), dP_ij = <dO_i, V_j>, dS_ij = p_ij (dP_ij - D_i), and
// accumulate dV_j += p_ij dO_i, dK_j += c dS_ij Q_i, dQ_i += c dS_ij K_j.
// No score or probability matrix is stored.
//
// gfx950 design (key-tile outer).  One workgroup owns 128 keys (32 per
// wave); each wave keeps its K and V rows in registers as MFMA B operands
// and its dK^T, dV^T accumulators in registers for the whole loop over
// query tiles.  Per query tile the workgroup stages Q, dO, L and D through
// double-buffered LDS.  Scores and dP are formed as S = Q K^T and
// dP = dO V^T with one key per lane column, so the accumulator registers
// holding P and dS are directly the B operand of dV^T += dO^T P and
// dK^T += Q^T dS; the dO^T and Q^T operands come from the row-major LDS
// tiles through transposed reads whose addresses follow the order in which
// a lane holds its query rows.  dS is written to LDS (key-major) and read
// back with transposed reads as the A operand of dQ = dS K, which the
// workgroup adds into an fp32 accumulator with hardware float atomics
// (coalesced: consecutive lanes hit consecutive d).  Fully masked query
// tiles are skipped; only partial ones are masked.
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
  static constexpr int KSTR = DP * ES + (BF16 ? 32 : 16);   // K tile (tr reads for dQ)
  static constexpr int QSTR = DP * ES + (BF16 ? 32 : 16);   // Q tile (row + tr reads)
  static constexpr int OSTR = DVP * ES + (BF16 ? 32 : 16);  // dO tile (row + tr reads)
  static constexpr int SSTR = BQ * ES + (BF16 ? 32 : 16);   // dS^T tile [key][q]
  static constexpr int KTILE = BK * KSTR;
  static constexpr int QTILE = BQ * QSTR;
  static constexpr int OTILE = BQ * OSTR;
  static constexpr int STILE = BK * SSTR;
  static constexpr int MWORDS = BK / 32;  // mask words per query row per key tile
  // Per buffer: Q tile, dO tile, L (base 2), D, mask words.
  static constexpr int BUF = QTILE + OTILE + BQ * 4 * 2 + BQ * MWORDS * 4;
  static constexpr int SMEM = KTILE + 2 * BUF + STILE;
  static constexpr int QCH = D * ES / 16;
  static constexpr int OCH = DV * ES / 16;
  static constexpr int QLD = (BQ * QCH + 255) / 256;
  static constexpr int OLD = (BQ * OCH + 255) / 256;
};

template <bool BF16, int D, int DV, int MASK>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdParams p) {
  using S = BwdShape<BF16, D, DV>;
  __shared__ __attribute__((aligned(16))) char smem[S::SMEM];
  char* Ks = smem;
  char* dSs = smem + S::KTILE + 2 * S::BUF;

  const int64_t logical = xcd_logical(blockIdx.x, p.grid_pad, p.total);
  if (logical < 0) return;
  const int64_t unit = logical / p.tk;
  const int kt = (int)(logical % p.tk);  // low key tiles (most causal work) first
  const int b = (int)(unit / p.H), h = (int)(unit % p.H);
  const int64_t n = p.n;
  const int64_t k0 = (int64_t)kt * S::BK;

  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int hh = lane / 32;
  const int g1 = (lane >> 4) & 1;
  const int klocal = 32 * w + (lane & 31);
  const int64_t key = k0 + klocal;
  const bool kvalid = key < n;

  const char* Qb = (const char*)p.Q + (b * p.sq[0] + h * p.sq[1]) * S::ES;
  const char* Kb = (const char*)p.K + (b * p.sk[0] + h * p.sk[1]) * S::ES;
  const char* Vb = (const char*)p.V + (b * p.sv[0] + h * p.sv[1]) * S::ES;
  const char* dOb = (const char*)p.dO + (b * p.so[0] + h * p.so[1]) * S::ES;
  const float* Lb = p.L + unit * n;
  const float* Db = p.Dv + unit * n;
  float* dQa = p.dQacc + unit * n * D;

  // Resident K tile in LDS (B operand of dQ), padded columns cleared.
  {
    constexpr int KCH = S::DP * S::ES / 16;
    for (int c = tid; c < S::BK * KCH; c += 256) {
      const int r = c / KCH, cc = c % KCH;
      const int64_t kr = k0 + r;
      u32x4 x = u32x4{0, 0, 0, 0};
      if (kr < n && cc * 16 < D * S::ES) x = *reinterpret_cast<const u32x4*>(Kb + kr * p.sk[2] * S::ES + cc * 16);
      *reinterpret_cast<u32x4*>(Ks + r * S::KSTR + cc * 16) = x;
    }
    // Clear padded columns of both Q / dO buffers once.
    if constexpr (S::DP != D || S::DVP != DV) {
      for (int bufi = 0; bufi < 2; ++bufi) {
        char* Qs = smem + S::KTILE + bufi * S::BUF;
        char* Os = Qs + S::QTILE;
        constexpr int qpc = (S::DP - D) * S::ES / 16, opc = (S::DVP - DV) * S::ES / 16;
        for (int c = tid; c < S::BQ * qpc; c += 256)
          *reinterpret_cast<u32x4*>(Qs + (c / qpc) * S::QSTR + D * S::ES + (c % qpc) * 16) = u32x4{0, 0, 0, 0};
        for (int c = tid; c < S::BQ * opc; c += 256)
          *reinterpret_cast<u32x4*>(Os + (c / opc) * S::OSTR + DV * S::ES + (c % opc) * 16) = u32x4{0, 0, 0, 0};
      }
    }
  }

  // Per-wave K and V rows as B operands (lane column = its key).
  typedef typename std::conditional<BF16, bf16x8, float>::type Frag;
  constexpr int NKF = D / S::KSTEP, NVF = DV / S::KSTEP;
  Frag kf[NKF], vf[NVF];
#pragma unroll
  for (int s = 0; s < NKF; ++s) {
    if constexpr (BF16)
      kf[s] = kvalid ? *reinterpret_cast<const bf16x8*>(Kb + (key * p.sk[2] + 16 * s + 8 * hh) * 2) : bf16x8{};
    else
      kf[s] = kvalid ? *reinterpret_cast<const float*>(Kb + (key * p.sk[2] + 2 * s + hh) * 4) : 0.f;
  }
#pragma unroll
  for (int s = 0; s < NVF; ++s) {
    if constexpr (BF16)
      vf[s] = kvalid ? *reinterpret_cast<const bf16x8*>(Vb + (key * p.sv[2] + 16 * s + 8 * hh) * 2) : bf16x8{};
    else
      vf[s] = kvalid ? *reinterpret_cast<const float*>(Vb + (key * p.sv[2] + 2 * s + hh) * 4) : 0.f;
  }

  f32x16 dk[S::NDB], dv[S::NVB];
#pragma unroll
  for (int i = 0; i < S::NDB; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < S::NVB; ++i) dv[i] = f32x16{};

  // Query-tile range and classification for this key tile.
  int qt_begin = 0;
  if constexpr (MASK == kMaskCausal) qt_begin = (int)(k0 / S::BQ);
  const uint8_t* map_col = nullptr;
  const uint32_t* mbase = nullptr;
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    map_col = p.map + mu * (int64_t)p.tq * p.tk + kt;
    mbase = p.mask + b * p.mask_sb + h * p.mask_sh;
  }
  auto tile_class = [&](int qt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return map_col[(int64_t)qt * p.tk];
    return classify_analytic(MASK, (int64_t)qt * S::BQ, S::BQ, k0, S::BK, n);
  };
  auto next_tile = [&](int qt) -> int {
    for (int t = qt + 1; t < p.tq; ++t)
      if (tile_class(t) != kTileEmpty) return t;
    return p.tq;
  };

  u32x4 qreg[S::QLD], oreg[S::OLD];
  float lreg = 0.f, dreg = 0.f;
  uint32_t mreg = 0;
  auto gload = [&](int qt) {
    const int64_t q0 = (int64_t)qt * S::BQ;
#pragma unroll
    for (int i = 0; i < S::QLD; ++i) {
      const int c = tid + i * 256;
      const int r = c / S::QCH, cc = c % S::QCH;
      const int64_t qq = q0 + r;
      qreg[i] = (c < S::BQ * S::QCH && qq < n)
                    ? *reinterpret_cast<const u32x4*>(Qb + qq * p.sq[2] * S::ES + cc * 16)
                    : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < S::OLD; ++i) {
      const int c = tid + i * 256;
      const int r = c / S::OCH, cc = c % S::OCH;
      const int64_t qq = q0 + r;
      oreg[i] = (c < S::BQ * S::OCH && qq < n)
                    ? *reinterpret_cast<const u32x4*>(dOb + qq * p.so[2] * S::ES + cc * 16)
                    : u32x4{0, 0, 0, 0};
    }
    if (tid < S::BQ) {
      const int64_t qq = q0 + tid;
      const float Lv = qq < n ? Lb[qq] : -INFINITY;
      // Rows with L = -inf (no allowed key, or past n) get +inf: p = exp2(s - inf) = 0.
      lreg = (Lv == -INFINITY) ? INFINITY : Lv * kLog2e;
      dreg = qq < n ? Db[qq] : 0.f;
    }
    if constexpr (MASK == kMaskBitmask) {
      if (tid < S::BQ * S::MWORDS) {
        const int r = tid / S::MWORDS, wi = tid % S::MWORDS;
        const int64_t qq = q0 + r;
        const int64_t wd = (k0 >> 5) + wi;
        mreg = (qq < n && wd * 32 < n) ? mbase[qq * p.mask_si + wd] : 0u;
      }
    }
  };
  auto lstore = [&](int bufi) {
    char* Qs = smem + S::KTILE + bufi * S::BUF;
    char* Os = Qs + S::QTILE;
    float* Ls = reinterpret_cast<float*>(Os + S::OTILE);
    float* Dsv = Ls + S::BQ;
    uint32_t* Ms = reinterpret_cast<uint32_t*>(Dsv + S::BQ);
#pragma unroll
    for (int i = 0; i < S::QLD; ++i) {
      const int c = tid + i * 256;
      if (c < S::BQ * S::QCH)
        *reinterpret_cast<u32x4*>(Qs + (c / S::QCH) * S::QSTR + (c % S::QCH) * 16) = qreg[i];
    }
#pragma unroll
    for (int i = 0; i < S::OLD; ++i) {
      const int c = tid + i * 256;
      if (c < S::BQ * S::OCH)
        *reinterpret_cast<u32x4*>(Os + (c / S::OCH) * S::OSTR + (c % S::OCH) * 16) = oreg[i];
    }
    if (tid < S::BQ) {
      Ls[tid] = lreg;
      Dsv[tid] = dreg;
    }
    if constexpr (MASK == kMaskBitmask) {
      if (tid < S::BQ * S::MWORDS) Ms[tid] = mreg;
    }
  };

  int qt = tile_class(qt_begin) != kTileEmpty ? qt_begin : next_tile(qt_begin);
  if (qt < p.tq) {
    gload(qt);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;

  while (qt < p.tq) {
    const int nq = next_tile(qt);
    const uint8_t cls = tile_class(qt);
    if (nq < p.tq) gload(nq);
    const int64_t q0 = (int64_t)qt * S::BQ;
    const char* Qs = smem + S::KTILE + buf * S::BUF;
    const char* Os = Qs + S::QTILE;
    const float* Ls = reinterpret_cast<const float*>(Os + S::OTILE);
    const float* Dsv = Ls + S::BQ;
    const uint32_t* Ms = reinterpret_cast<const uint32_t*>(Dsv + S::BQ);

    bool active = true;
    if constexpr (MASK == kMaskCausal) active = (k0 + 32 * w) <= (q0 + S::BQ - 1);  // wave-uniform
    if (active) {
#pragma unroll
      for (int qb = 0; qb < S::NQB; ++qb) {
        // S = Q K^T and dP = dO V^T for 32 query rows x this wave's 32 keys.
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < NKF; ++s) {
          if constexpr (BF16) {
            bf16x8 a = lds_read_b128(Qs, (32 * qb + (lane & 31)) * S::QSTR + (16 * s + 8 * hh) * 2);
            sc = mfma_bf16(a, kf[s], sc);
          } else {
            float a = *reinterpret_cast<const float*>(Qs + (32 * qb + (lane & 31)) * S::QSTR + (2 * s + hh) * 4);
            sc = mfma_f32(a, kf[s], sc);
          }
        }
#pragma unroll
        for (int s = 0; s < NVF; ++s) {
          if constexpr (BF16) {
            bf16x8 a = lds_read_b128(Os, (32 * qb + (lane & 31)) * S::OSTR + (16 * s + 8 * hh) * 2);
            dp = mfma_bf16(a, vf[s], dp);
          } else {
            float a = *reinterpret_cast<const float*>(Os + (32 * qb + (lane & 31)) * S::OSTR + (2 * s + hh) * 4);
            dp = mfma_f32(a, vf[s], dp);
          }
        }
        // P = exp2(s c log2e - L log2e); dS = P (dP - D).  Register r holds
        // query row 32 qb + 8 (r/4) + 4 hh + r%4 of the tile.
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = 32 * qb + 8 * g + 4 * hh;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + ql);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dsv + ql);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pv = fast_exp2(sc[r] * p.scale2 - l4[e]);
            if (cls == kTilePartial) {
              const int64_t qq = q0 + ql + e;
              bool ok = kvalid;
              if constexpr (MASK == kMaskCausal) ok = ok && key <= qq;
              if constexpr (MASK == kMaskBitmask)
                ok = ok && ((Ms[(ql + e) * S::MWORDS + (klocal >> 5)] >> (klocal & 31)) & 1u);
              pv = ok ? pv : 0.f;
            }
            sc[r] = pv;
            dp[r] = pv * (dp[r] - d4[e]);
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS.
        if constexpr (BF16) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 pb = pack8(sc, 8 * ks);
            const bf16x8 sb = pack8(dp, 8 * ks);
            const int kr = 32 * qb + 16 * ks + 4 * hh;
#pragma unroll
            for (int vb = 0; vb < S::NVB; ++vb) {
              const int n0 = vb * 32 + 16 * g1;
              i16x4 lo = lds_read_tr(Os, tr_addr(lane, kr, n0, S::OSTR));
              i16x4 hi = lds_read_tr(Os, tr_addr(lane, kr + 8, n0, S::OSTR));
              dv[vb] = mfma_bf16(join_tr(lo, hi), pb, dv[vb]);
            }
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              const int n0 = db * 32 + 16 * g1;
              i16x4 lo = lds_read_tr(Qs, tr_addr(lane, kr, n0, S::QSTR));
              i16x4 hi = lds_read_tr(Qs, tr_addr(lane, kr + 8, n0, S::QSTR));
              dk[db] = mfma_bf16(join_tr(lo, hi), sb, dk[db]);
            }
          }
          // dS^T -> LDS (key-major): 4 consecutive query rows per store.
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int ql = 32 * qb + 8 * g + 4 * hh;
            u32x2 pk{pack_bf16x2(dp[4 * g], dp[4 * g + 1]), pack_bf16x2(dp[4 * g + 2], dp[4 * g + 3])};
            *reinterpret_cast<u32x2*>(dSs + klocal * S::SSTR + ql * 2) = pk;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
            for (int vb = 0; vb < S::NVB; ++vb) {
              float a = *reinterpret_cast<const float*>(Os + ql * S::OSTR + (vb * 32 + (lane & 31)) * 4);
              dv[vb] = mfma_f32(a, sc[r], dv[vb]);
            }
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              float a = *reinterpret_cast<const float*>(Qs + ql * S::QSTR + (db * 32 + (lane & 31)) * 4);
              dk[db] = mfma_f32(a, dp[r], dk[db]);
            }
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int ql = 32 * qb + 8 * g + 4 * hh;
            *reinterpret_cast<f32x4*>(dSs + klocal * S::SSTR + ql * 4) =
                f32x4{dp[4 * g], dp[4 * g + 1], dp[4 * g + 2], dp[4 * g + 3]};
          }
        }
      }
    } else {
      // All of this wave's keys are masked for the tile: its dS rows are zero.
      if constexpr (BF16) {
        for (int c = lane; c < 32 * S::BQ / 8; c += kWave) {
          const int r = c / (S::BQ / 8), cc = c % (S::BQ / 8);
          *reinterpret_cast<u32x4*>(dSs + (32 * w + r) * S::SSTR + cc * 16) = u32x4{0, 0, 0, 0};
        }
      } else {
        for (int c = lane; c < 32 * S::BQ / 4; c += kWave) {
          const int r = c / (S::BQ / 4), cc = c % (S::BQ / 4);
          *reinterpret_cast<u32x4*>(dSs + (32 * w + r) * S::SSTR + cc * 16) = u32x4{0, 0, 0, 0};
        }
      }
    }
    __syncthreads();  // dS of all 128 keys in LDS

    // dQ (this query tile, all d) += dS K over the workgroup's 128 keys.
    for (int blk = w; blk < S::NQB * S::NDB; blk += S::NW) {
      const int qb = blk % S::NQB, db = blk / S::NQB;
      f32x16 acc = f32x16{};
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < S::BK / 16; ++ks) {
          const int kr = 16 * ks + 8 * hh;
          i16x4 alo = lds_read_tr(dSs, tr_addr(lane, kr, 32 * qb + 16 * g1, S::SSTR));
          i16x4 ahi = lds_read_tr(dSs, tr_addr(lane, kr + 4, 32 * qb + 16 * g1, S::SSTR));
          i16x4 blo = lds_read_tr(Ks, tr_addr(lane, kr, 32 * db + 16 * g1, S::KSTR));
          i16x4 bhi = lds_read_tr(Ks, tr_addr(lane, kr + 4, 32 * db + 16 * g1, S::KSTR));
          acc = mfma_bf16(join_tr(alo, ahi), join_tr(blo, bhi), acc);
        }
      } else {
#pragma unroll 8
        for (int ks = 0; ks < S::BK / 2; ++ks) {
          const int kr = 2 * ks + hh;
          float a = *reinterpret_cast<const float*>(dSs + kr * S::SSTR + (32 * qb + (lane & 31)) * 4);
          float bb = *reinterpret_cast<const float*>(Ks + kr * S::KSTR + (32 * db + (lane & 31)) * 4);
          acc = mfma_f32(a, bb, acc);
        }
      }
      const int dcol = 32 * db + (lane & 31);
      if (dcol < D) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t qq = q0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (qq < n) unsafeAtomicAdd(dQa + qq * D + dcol, acc[r]);
        }
      }
    }

    if (nq < p.tq) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    qt = nq;
  }

  // Epilogue: dK = c dK^T, dV = dV^T (lane = key; 4 consecutive columns per store).
  if (kvalid) {
    char* dKp = (char*)p.dK + (b * p.sk[0] + h * p.sk[1] + key * p.sk[2]) * S::ES;
    char* dVp = (char*)p.dV + (b * p.sv[0] + h * p.sv[1] + key * p.sv[2]) * S::ES;
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
          const float x0 = dv[vb][4 * g], x1 = dv[vb][4 * g + 1];
          const float x2 = dv[vb][4 * g + 2], x3 = dv[vb][4 * g + 3];
          if constexpr (BF16)
            *reinterpret_cast<u32x2*>(dVp + c0 * 2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          else
            *reinterpret_cast<f32x4*>(dVp + c0 * 4) = f32x4{x0, x1, x2, x3};
        }
      }
  }
}

template <bool BF16, int D, int DV, int MASK>
static int launch_one(const BwdParams& p, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kernel<BF16, D, DV, MASK>), dim3((unsigned)p.grid_pad), dim3(256), 0, st, p);
  return (int)hipGetLastError();
}

template <bool BF16, int D, int DV>
static int launch_mask(const BwdParams& p, int mask_mode, hipStream_t st) {
  switch (mask_mode) {
    case kMaskNone: return launch_one<BF16, D, DV, kMaskNone>(p, st);
    case kMaskCausal: return launch_one<BF16, D, DV, kMaskCausal>(p, st);
    default: return launch_one<BF16, D, DV, kMaskBitmask>(p, st);
  }
}

template <bool BF16>
static int launch_dims(const BwdParams& p, int d, int v, int mask_mode, hipStream_t st) {
  if (d == 64 && v == 64) return launch_mask<BF16, 64, 64>(p, mask_mode, st);
  if (d == 80 && v == 80) return launch_mask<BF16, 80, 80>(p, mask_mode, st);
  if (d == 128 && v == 128) return launch_mask<BF16, 128, 128>(p, mask_mode, st);
  if (d == 64 && v == 128) return launch_mask<BF16, 64, 128>(p, mask_mode, st);
  return (int)hipErrorInvalidValue;
}

int launch_bwd(const BwdParams& p, int bf16, int d, int v, int mask_mode, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return bf16 ? launch_dims<true>(p, d, v, mask_mode, st) : launch_dims<false>(p, d, v, mask_mode, st);
}

}  // namespace eta
