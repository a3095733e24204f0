// Forward kernel: exact attention with an online softmax over key tiles.
//
// Method (ob1 page, part 1; trentorch exercise, hint and constraints;
// maitreyasuin post, the tiled forward): per query row keep a running
// maximum m, a running denominator l and the unnormalised output; for each
// key tile rescale l and the output by exp(m_old - m_new) when the maximum
// grows, add exp(s - m) and its product with V; normalise once at the end
// and keep L = m + ln l.  Tiles whose intersection with every row's allowed
// set is empty are skipped and only partially allowed tiles are masked (ob1
// page, part 3; alphabetamath page, forward step 2).
//
// gfx950 design.  One workgroup = 4 waves = 128 query rows; each wave owns
// 32 rows and two workgroups share a CU (two waves per SIMD), so one wave's
// softmax overlaps the other's MFMAs.  Scores are formed transposed,
// S^T = K Q^T, with the wave's Q rows held in registers as the MFMA B
// operand, so every lane owns one query column: the row max and row sum are
// in-lane reductions plus one permlane32 swap, and the rescale factor is a
// per-lane scalar.  The output accumulator is kept transposed too,
// O^T += V^T P^T: P^T comes straight from the score registers (bf16 RNE) and
// V^T from the row-major V tile through transposed LDS reads
// (ds_read_b64_tr_b16) whose addresses follow the order in which a lane
// holds its keys, so no shuffle is needed.  K and V tiles of 64 keys are
// loaded with buffer loads (rows past n read as zero) into registers while
// the previous tile is computed, then stored to a second, XOR-swizzled LDS
// buffer.  The maximum is raised lazily (only when exceeded by more than
// 2^8), which leaves O and L unchanged because softmax is shift-invariant.
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {

template <bool BF16, int D, int DV>
struct FwdShape {
  static constexpr int NW = 4;
  static constexpr int BQ = kFwdBq;
  static constexpr int BK = kFwdBk;
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int KSTEP = BF16 ? 16 : 2;  // contraction per MFMA
  static constexpr int DVP = (DV + 31) / 32 * 32;
  static constexpr int NVB = DVP / 32;
  static constexpr int NKB = BK / 32;
  static constexpr int KCH = D * ES / 16;   // 16-byte chunks per K row
  static constexpr int VCH = DV * ES / 16;  // 16-byte chunks per V row (loaded)
  using KT = Swz<KCH>;                      // K tile layout in LDS
  using VT = Swz<DVP * ES / 16>;            // V tile layout in LDS (padded columns)
  static constexpr int KTILE = BK * KT::kStride;
  static constexpr int VTILE = BK * VT::kStride;
  static constexpr int KLD = (BK * KCH + NW * kWave - 1) / (NW * kWave);
  static constexpr int VLD = (BK * VCH + NW * kWave - 1) / (NW * kWave);
  static constexpr int NQF = D / KSTEP;  // Q fragments per lane
  static constexpr int SMEM = 2 * (KTILE + VTILE);
};

// Lazy rescaling: the reference maximum m is raised only when a tile's max
// exceeds it by more than this (base-2 units).  Any reference value gives
// the same O and L (softmax is shift-invariant); this bound keeps the
// unnormalised weights <= 2^8.
constexpr float kRescaleSlack = 8.0f;
// Bound on a lane's sum of 32 weights below which none of them exceeds
// 2^(kRescaleSlack - 1) (the pipelined forward's test for keeping its
// reference max without computing the row max).
constexpr float kSpecBound = 128.0f;

// DROP: dropout on the weights (kern_common.h keep decisions): the PV
// product takes the kept weights only, the normaliser and L stay those of
// the undropped softmax, and O is scaled by 1 / P(keep).
template <bool BF16, int D, int DV, int MASK, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(FwdParams p) {
  using S = FwdShape<BF16, D, DV>;
  __shared__ __attribute__((aligned(16))) char smem[S::SMEM];

  const int64_t logical = xcd_logical(blockIdx.x, p.grid_pad, p.total);
  if (logical < 0) return;
  const int unit = (int)(logical / p.tq);
  const int qt = p.tq - 1 - (int)(logical % p.tq);  // heaviest causal tiles first
  const int b = unit / p.H, h = unit % p.H;
  const int n = (int)p.n, nk = (int)p.nk, coff = (int)p.coff;  // query rows, key rows, causal offset
  const int q0 = qt * S::BQ;

  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int hh = lane >> 5;        // half-wave
  const int g1 = (lane >> 4) & 1;  // 16-lane group within the half
  const int q = q0 + 32 * w + (lane & 31);
  const bool qvalid = q < n;

  // Buffer resources: rows at or past n read as zero.
  const int qrow = (int)p.sq[2] * S::ES, krow = (int)p.sk[2] * S::ES, vrow = (int)p.sv[2] * S::ES;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * S::ES;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * S::ES;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * S::ES;

  // Q fragments (B operand of S^T = K Q^T).  For c < 0 the rows are negated
  // (exact) and |c| is used, so the tile max is taken on raw scores.  |c|
  // log2(e) is clamped to >= 1e-30: for c = 0 every score maps to
  // exp2(~1e-24) = 1.0f exactly, while masked scores (-inf) stay -inf.
  const bool neg = p.scale2 < 0.f;
  const float scale2 = fmaxf(fabsf(p.scale2), 1e-30f);
  typedef typename std::conditional<BF16, bf16x8, float>::type QFrag;
  QFrag qf[S::NQF];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb, (int64_t)n * qrow);
    const int qoff = q * qrow;
#pragma unroll
    for (int ks = 0; ks < S::NQF; ++ks) {
      if constexpr (BF16) {
        u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (16 * ks + 8 * hh) * 2, 0, 0);
        if (neg) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qf[ks] = __builtin_bit_cast(bf16x8, x);
      } else {
        const float x =
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rq, qoff + (2 * ks + hh) * 4, 0, 0));
        qf[ks] = neg ? -x : x;
      }
    }
  }

  // Key-tile range and classification.
  int kt_end = p.tk;
  if constexpr (MASK == kMaskCausal) {
    const int k_hi = (q0 + S::BQ < n ? q0 + S::BQ : n) - 1 + coff;  // last key any row allows
    kt_end = k_hi < 0 ? 0 : (k_hi / S::BK + 1 < p.tk ? k_hi / S::BK + 1 : p.tk);
  }
  const uint8_t* map_row = nullptr;
  const uint32_t* mrow = nullptr;
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    map_row = p.map + (mu * p.tq + qt) * (int64_t)p.tk;
    mrow = p.mask + b * p.mask_sb + h * p.mask_sh + (int64_t)(qvalid ? q : 0) * p.mask_si;
  }
  auto tile_class = [&](int kt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return map_row[kt];
    return classify_analytic(MASK, q0, S::BQ, (int64_t)kt * S::BK, S::BK, n, nk, coff);
  };
  // Next tile with an allowed pair (none/causal: every tile in [0, kt_end) has one).
  auto next_tile = [&](int kt) -> int {
    if constexpr (MASK != kMaskBitmask) return kt + 1;
    for (int k = kt + 1; k < kt_end; ++k)
      if (tile_class(k) != kTileEmpty) return k;
    return kt_end;
  };

  // Zero the padded value columns of both V buffers once (only when DV % 32).
  if constexpr (S::DVP != DV) {
    constexpr int padc = (S::DVP - DV) * S::ES / 16;
    for (int c = tid; c < 2 * S::BK * padc; c += 256) {
      const int bf = c / (S::BK * padc), r = (c / padc) % S::BK, cc = c % padc;
      *reinterpret_cast<u32x4*>(smem + bf * (S::KTILE + S::VTILE) + S::KTILE + S::VT::off(r, S::VCH + cc)) =
          u32x4{0, 0, 0, 0};
    }
  }

  // Staging: thread chunk c = tid + 256 i covers row c / CH, 16-byte column c % CH.
  u32x4 kreg[S::KLD], vreg[S::VLD];
  auto gload = [&](int kt) {
    const int k0 = kt * S::BK;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb + (int64_t)k0 * krow, (int64_t)(nk - k0) * krow);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vb + (int64_t)k0 * vrow, (int64_t)(nk - k0) * vrow);
#pragma unroll
    for (int i = 0; i < S::KLD; ++i) {
      const int c = tid + i * 256;
      if (S::BK * S::KCH % 256 == 0 || c < S::BK * S::KCH)
        kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (c / S::KCH) * krow + (c % S::KCH) * 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < S::VLD; ++i) {
      const int c = tid + i * 256;
      if (S::BK * S::VCH % 256 == 0 || c < S::BK * S::VCH)
        vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, (c / S::VCH) * vrow + (c % S::VCH) * 16, 0, 0);
    }
  };
  auto lstore = [&](int bf) {
    char* kt_s = smem + bf * (S::KTILE + S::VTILE);
    char* vt_s = kt_s + S::KTILE;
#pragma unroll
    for (int i = 0; i < S::KLD; ++i) {
      const int c = tid + i * 256;
      if (S::BK * S::KCH % 256 == 0 || c < S::BK * S::KCH)
        *reinterpret_cast<u32x4*>(kt_s + S::KT::off(c / S::KCH, c % S::KCH)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < S::VLD; ++i) {
      const int c = tid + i * 256;
      if (S::BK * S::VCH % 256 == 0 || c < S::BK * S::VCH)
        *reinterpret_cast<u32x4*>(vt_s + S::VT::off(c / S::VCH, c % S::VCH)) = vreg[i];
    }
  };

  // Running state for this lane's query row (both half-waves hold it).
  // l_run sums the fp32 weights (for L); l_use sums the weights as the PV
  // product consumes them (bf16-rounded on the bf16 path), so O is normalised
  // by the weights actually used.
  float m_run = -INFINITY;
  float l_run = 0.f, l_use = 0.f;
  f32x16 o[S::NVB];
#pragma unroll
  for (int vb = 0; vb < S::NVB; ++vb) o[vb] = f32x16{};

  int kt = 0, ntiles = 0;
  if (MASK == kMaskBitmask && kt < kt_end && tile_class(kt) == kTileEmpty) kt = next_tile(kt);
  if (kt < kt_end) {
    gload(kt);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  const int wave_k_hi = q0 + 32 * w + 31 + coff;  // last key this wave's rows can allow

  while (kt < kt_end) {
    const int kn = next_tile(kt);
    const uint8_t cls = tile_class(kt);
    if (kn < kt_end) gload(kn);
    const int k0 = kt * S::BK;
    const char* Ks = smem + buf * (S::KTILE + S::VTILE);
    const char* Vs = Ks + S::KTILE;

    bool active = true;
    if constexpr (MASK == kMaskCausal) active = k0 <= wave_k_hi;  // wave-uniform
    if (active) {
      // S^T = K Q^T for NKB blocks of 32 keys.
      f32x16 s[S::NKB];
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < S::NQF; ++ks) {
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb) {
          if constexpr (BF16) {
            const bf16x8 a = lds_read_b128(Ks, S::KT::off(32 * kb + (lane & 31), 2 * ks + hh));
            s[kb] = mfma_bf16(a, qf[ks], s[kb]);
          } else {
            const float a =
                *reinterpret_cast<const float*>(Ks + S::KT::off_dword(32 * kb + (lane & 31), 2 * ks + hh));
            s[kb] = mfma_f32(a, qf[ks], s[kb]);
          }
        }
      }
      // Mask partial tiles; tile row max on raw scores (scale2 > 0).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb) {
        if (cls == kTilePartial) {
          uint32_t word = 0xFFFFFFFFu;
          if constexpr (MASK == kMaskBitmask) {
            if (qvalid && k0 + 32 * kb < nk) word = mrow[(k0 + 32 * kb) >> 5];
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int key = k0 + kk;
            bool ok = key < nk;
            if constexpr (MASK == kMaskCausal) ok = ok && key <= q + coff;
            if constexpr (MASK == kMaskBitmask) ok = ok && ((word >> (kk & 31)) & 1u);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = max_halves(mx) * scale2;  // base-2 units; -inf stays -inf (scale2 > 0)
      // Raise the reference max only when it is exceeded by more than the
      // slack.  The branch is taken when any lane needs it, but each lane
      // decides for its own row (others keep m and get alpha = 1 exactly), so
      // a row's result never depends on the other rows of the wave.
      const bool raise = mx > m_run + kRescaleSlack;
      if (__ballot(raise) != 0) {
        const float m_new = raise ? fmaxf(m_run, mx) : m_run;
        const float alpha = (!raise || m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
        l_use *= alpha;
#pragma unroll
        for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[vb][r] *= alpha;
        m_run = m_new;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      u32x4 pk[S::NKB][2];  // bf16 path: weights packed in pairs, one PV operand per 16 keys
      // Dropout: registers 4g..4g+3 of block kb hold 4 consecutive keys of this
      // lane's row; the quad's lanes hold rows 4a..4a+3, so lane g of the quad
      // draws group g for all four rows (keep_mask16) and each lane takes its
      // row's nibble of every group.
      uint32_t keep4[S::NKB][4];
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb) {
        if constexpr (DROP) {
          const uint32_t e = (uint32_t)lane & 3u;
          const uint32_t m = keep_mask16(p.drop.seed_lo, p.drop.seed_hi, p.drop.p8,
                                         (uint32_t)(k0 + 32 * kb + 8 * (int)e + 4 * hh) >> 2, (uint32_t)q >> 2,
                                         (uint32_t)unit, false);
          keep4[kb][0] = (quad_bcast<0>(m) >> (4 * e)) & 0xFu;
          keep4[kb][1] = (quad_bcast<1>(m) >> (4 * e)) & 0xFu;
          keep4[kb][2] = (quad_bcast<2>(m) >> (4 * e)) & 0xFu;
          keep4[kb][3] = (quad_bcast<3>(m) >> (4 * e)) & 0xFu;
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) keep4[kb][g] = 0xFu;
        }
      }
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const uint32_t keep = keep4[kb][r >> 2];
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], scale2, neg_m));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], scale2, neg_m));
          l_run += p0 + p1;
          const bool z0 = (keep >> (r & 3)) & 1u, z1 = (keep >> ((r + 1) & 3)) & 1u;
          if constexpr (BF16) {
            const uint32_t u = pack_bf16x2(p0, p1);
            pk[kb][r / 8][(r / 2) % 4] = DROP ? (u & ((z0 ? 0xFFFFu : 0u) | (z1 ? 0xFFFF0000u : 0u))) : u;
            l_use = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u), ones_bf16x2(), l_use, false);
          } else {
            s[kb][r] = (!DROP || z0) ? p0 : 0.f;
            s[kb][r + 1] = (!DROP || z1) ? p1 : 0.f;
          }
        }
      if constexpr (!BF16) l_use = l_run;

      // O^T += V^T P^T.
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < S::BK / 16; ++ks) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[ks / 2][ks % 2]);
#pragma unroll
          for (int vb = 0; vb < S::NVB; ++vb) {
            const int n0 = vb * 32 + 16 * g1;
            const i16x4 lo = lds_read_tr(Vs, S::VT::tr(lane, 16 * ks + 4 * hh, n0));
            const i16x4 hi = lds_read_tr(Vs, S::VT::tr(lane, 16 * ks + 8 + 4 * hh, n0));
            o[vb] = mfma_bf16(join_tr(lo, hi), pb, o[vb]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
            for (int vb = 0; vb < S::NVB; ++vb) {
              const float a = *reinterpret_cast<const float*>(Vs + S::VT::off_dword(kk, vb * 32 + (lane & 31)));
              o[vb] = mfma_f32(a, s[kb][r], o[vb]);
            }
          }
      }
    }
    if (kn < kt_end) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    kt = kn;
    ++ntiles;
  }
  count_tiles(p.tile_count, ntiles);

  // Epilogue: O = acc / l, L = (m + log2 l) ln 2.
  const float l_tot = sum_halves(l_run);
  const float l_norm = sum_halves(l_use);
  const float inv = l_norm > 0.f ? (DROP ? p.drop.keep_inv : 1.f) / l_norm : 0.f;
  if (qvalid) {
    const int64_t obase = (int64_t)b * p.so[0] + (int64_t)h * p.so[1] + (int64_t)q * p.so[2];
#pragma unroll
    for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int vd = vb * 32 + 8 * g + 4 * hh;
        if (vd < DV) {
          const float x0 = o[vb][4 * g] * inv, x1 = o[vb][4 * g + 1] * inv;
          const float x2 = o[vb][4 * g + 2] * inv, x3 = o[vb][4 * g + 3] * inv;
          if constexpr (BF16) {
            const u32x2 pk2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
            *reinterpret_cast<u32x2*>((char*)p.O + (obase + vd) * 2) = pk2;
          } else {
            *reinterpret_cast<f32x4*>((char*)p.O + (obase + vd) * 4) = f32x4{x0, x1, x2, x3};
          }
        }
      }
    if (hh == 0) {
      const float Lv = (m_run == -INFINITY || l_tot <= 0.f) ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
      p.L[(int64_t)unit * n + q] = Lv;
    }
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined bf16 forward (d, v in {64, 128}).
//
// Same tiling, state and arithmetic as fwd_kernel, scheduled differently:
// the scores of key tile j+1 are formed on the matrix cores while the
// vector ALUs run the softmax of tile j, and the PV product of tile j runs
// beside the row max of tile j+1; the instruction order is pinned (one MFMA,
// its LDS reads issued ahead, a slice of VALU work).  K and V tiles go from
// HBM straight into padded LDS rows (buffer_load ... lds), so no registers
// are spent on staging and every LDS read address is a per-lane base plus a
// constant; K and V have two buffers each: K_{j+2} and V_{j+1} stream in
// while tile j is consumed.  O is normalised by the fp32 sum of the weights
// (the one L is taken from); the PV product uses their bf16 roundings.
// Dropout (DROP): the PV product takes P o Z and O is scaled by 1 / P(keep),
// with the keep decisions Z of kern_common.h regenerated per tile.
// ---------------------------------------------------------------------------
template <int D, int DV>
struct FwdPipeShape {
  static constexpr int BQ = kFwdBq, BK = kFwdBk, NW = 4;
  static constexpr int NQF = D / 16;   // Q fragments per lane (16 dims each)
  static constexpr int NVB = DV / 32;  // 32-column blocks of the output
  static constexpr int NKB = BK / 32;  // 32-key blocks of a tile
  using KT = PadTile<D * 2, 16>;   // b128 row reads
  using VT = PadTile<DV * 2, 64>;  // transposed reads
  static constexpr int KS = KT::kStride, VS = VT::kStride;
  static constexpr int KTILE = BK * KS, VTILE = BK * VS;
  static constexpr int KWINS = KTILE / 1024, VWINS = VTILE / 1024;  // 1 KB fill windows per tile
  static constexpr int KWIN = (KWINS + NW - 1) / NW, VWIN = (VWINS + NW - 1) / NW;  // per wave (max)
  static_assert(KTILE % 1024 == 0 && VTILE % 1024 == 0, "whole fill windows");
  static_assert(KWIN + VWIN <= (D / 16) * (BK / 32), "one copy per first-phase MFMA at most");
};

template <int D, int DV, int MASK, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_pipe_kernel(FwdParams p) {
  using S = FwdPipeShape<D, DV>;
  // Four distinct LDS objects, so that the compiler can tell reads of one
  // buffer from the direct fills in flight into another (no false waits).
  __shared__ __attribute__((aligned(1024))) char kbuf0[S::KTILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[S::KTILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[S::VTILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[S::VTILE];
  __shared__ __attribute__((aligned(1024))) char spare[1024];  // target of the copies a wave has no window for

  const int64_t logical0 = xcd_logical(blockIdx.x, p.grid_pad, p.total);
  if (logical0 < 0) return;
  const int split = (int)(logical0 % p.splits);  // key-range split (0 when not splitting)
  const int64_t logical = logical0 / p.splits;
  const int unit = (int)(logical / p.tq);
  const int qt = p.tq - 1 - (int)(logical % p.tq);  // heaviest causal tiles first
  const int b = unit / p.H, h = unit % p.H;
  const int n = (int)p.n, nk = (int)p.nk, coff = (int)p.coff;  // query rows, key rows, causal offset
  const int q0 = qt * S::BQ;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int g1 = (lane >> 4) & 1;
  const int q = q0 + 32 * w + (lane & 31);
  const bool qvalid = q < n;

  const int qrow = (int)p.sq[2] * 2, krow = (int)p.sk[2] * 2, vrow = (int)p.sv[2] * 2;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * 2;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * 2;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * 2;

  // Q fragments as the B operand of S^T = K Q^T (negated rows for c < 0;
  // |c| log2 e clamped to >= 1e-30, as in fwd_kernel).
  const bool neg = p.scale2 < 0.f;
  const float scale2 = fmaxf(fabsf(p.scale2), 1e-30f);
  bf16x8 qf[S::NQF];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb, (int64_t)n * qrow);
    const int qoff = q * qrow;
#pragma unroll
    for (int ks = 0; ks < S::NQF; ++ks) {
      u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (16 * ks + 8 * hh) * 2, 0, 0);
      if (neg) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  int kt_end = p.tk;
  if constexpr (MASK == kMaskCausal) {
    const int k_hi = (q0 + S::BQ < n ? q0 + S::BQ : n) - 1 + coff;  // last key any row allows
    kt_end = k_hi < 0 ? 0 : (k_hi / S::BK + 1 < p.tk ? k_hi / S::BK + 1 : p.tk);
  }
  const uint8_t* map_row = nullptr;
  const uint32_t* mrow = nullptr;
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    map_row = p.map + (mu * p.tq + qt) * (int64_t)p.tk;
    mrow = p.mask + b * p.mask_sb + h * p.mask_sh + (int64_t)(qvalid ? q : 0) * p.mask_si;
  }
  auto tile_class = [&](int kt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return map_row[kt];
    return classify_analytic(MASK, q0, S::BQ, (int64_t)kt * S::BK, S::BK, n, nk, coff);
  };
  auto next_tile = [&](int kt) -> int {
    if constexpr (MASK != kMaskBitmask) return kt + 1;
    for (int k = kt + 1; k < kt_end; ++k)
      if (tile_class(k) != kTileEmpty) return k;
    return kt_end;
  };

  // Per-lane source offsets of this wave's 1 KB fill windows w, w + 4, ...
  // (fixed per tile).
  int koff[S::KWIN], voff[S::VWIN];
#pragma unroll
  for (int i = 0; i < S::KWIN; ++i) koff[i] = S::KT::fill_src((w + S::NW * i) * 1024 + 16 * lane, krow);
#pragma unroll
  for (int i = 0; i < S::VWIN; ++i) voff[i] = S::VT::fill_src((w + S::NW * i) * 1024 + 16 * lane, vrow);
  const __amdgpu_buffer_rsrc_t rnone = make_rsrc(Kb, 0);
  const int kmax_rows = 0x7FFFFFFF / krow, vmax_rows = 0x7FFFFFFF / vrow;
  auto fill_k = [&](int kt, char* buf) {
    const int k0 = kt * S::BK;
    const __amdgpu_buffer_rsrc_t r = make_rsrc_rows(Kb + (int64_t)k0 * krow, nk - k0, krow, kmax_rows);
#pragma unroll
    for (int i = 0; i < S::KWIN; ++i)
      if (S::KWINS % S::NW == 0 || w + S::NW * i < S::KWINS) dma16(r, buf + (w + S::NW * i) * 1024, koff[i]);
  };
  auto fill_v = [&](int kt, char* buf) {
    const int k0 = kt * S::BK;
    const __amdgpu_buffer_rsrc_t r = make_rsrc_rows(Vb + (int64_t)k0 * vrow, nk - k0, vrow, vmax_rows);
#pragma unroll
    for (int i = 0; i < S::VWIN; ++i)
      if (S::VWINS % S::NW == 0 || w + S::NW * i < S::VWINS) dma16(r, buf + (w + S::NW * i) * 1024, voff[i]);
  };
  // Read bases: K row (lane % 32), chunk hh; V^T slice rows 4 hh + i / 4,
  // columns 16 g1 + 4 (i % 4) of a 16-lane group's transposed read.
  const int kbase = (lane & 31) * S::KS + 16 * hh;
  const int vbase = (4 * hh + ((lane & 15) >> 2)) * S::VS + (16 * g1 + 4 * (lane & 3)) * 2;

  // V rows past nk are multiplied by zero weights: when the last key tile is
  // partial, clear both V buffers once so that they never hold non-finite bit
  // patterns.  With nk a multiple of the tile height every fill writes every
  // row that is read.
  if (nk % S::BK != 0) {
    for (int c = tid; c < S::VTILE / 16; c += 256) {
      reinterpret_cast<u32x4*>(vbuf0)[c] = u32x4{0, 0, 0, 0};
      reinterpret_cast<u32x4*>(vbuf1)[c] = u32x4{0, 0, 0, 0};
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  float neg_m = 0.f;  // exponent offset of the weights: -m_run, 0 while m_run = -inf
  float spec_lim = 0.f;  // kSpecBound, 0 while m_run = -inf (any weight then takes the exact path)
  f32x16 o[S::NVB];
#pragma unroll
  for (int vb = 0; vb < S::NVB; ++vb) o[vb] = f32x16{};

  // S^T (this wave's 32 queries x 64 keys) of the K tile in `kb_s`.
  auto scores = [&](f32x16 (&sc)[S::NKB], const char* ks_s) {
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb) sc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < S::NQF; ++ks)
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb)
        sc[kb] = mfma_bf16(lds_read_b128(ks_s, kbase + 32 * kb * S::KS + 32 * ks), qf[ks], sc[kb]);
  };

  // Masking of a partially allowed tile's scores (keys past nk, causal, bitmask).
  auto mask_tile = [&](f32x16 (&sc)[S::NKB], int kt) {
    const int k0 = kt * S::BK;
    if constexpr (MASK == kMaskBitmask) {
      if (k0 + S::BK <= nk) {  // every key of the tile exists: the word's bit alone decides
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb) {
          const uint32_t word = qvalid ? mrow[(k0 + 32 * kb) >> 5] : 0xFFFFFFFFu;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
            // All ones iff allowed; disallowed scores become -inf (bit select).
            const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)word, (uint32_t)kk, 1u);
            sc[kb][r] = __uint_as_float((__float_as_uint(sc[kb][r]) & keep) | (0xFF800000u & ~keep));
          }
        }
        return;
      }
    }
    if constexpr (MASK == kMaskCausal) {
      if (k0 + S::BK <= nk) {  // every key of the tile exists: key <= q + coff alone decides
        const int lim = q + coff - k0 - 4 * hh;  // register offset kk - 4 hh must not exceed it
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sc[kb][r] = 32 * kb + 8 * (r >> 2) + (r & 3) <= lim ? sc[kb][r] : -INFINITY;
        return;
      }
    }
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb) {
      uint32_t word = 0xFFFFFFFFu;
      if constexpr (MASK == kMaskBitmask) {
        if (qvalid && k0 + 32 * kb < nk) word = mrow[(k0 + 32 * kb) >> 5];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int key = k0 + kk;
        bool ok = key < nk;
        if constexpr (MASK == kMaskCausal) ok = ok && key <= q + coff;
        if constexpr (MASK == kMaskBitmask) ok = ok && ((word >> (kk & 31)) & 1u);
        sc[kb][r] = ok ? sc[kb][r] : -INFINITY;
      }
    }
  };
  // Row max of a tile (base-2 units) and the lazy-rescale decision it implies:
  // the reference max is raised only when exceeded by more than the slack;
  // each lane decides for its own row.
  float m_new = -INFINITY, alpha = 1.f;
  bool raise = false;
  auto row_max = [&](const f32x16 (&sc)[S::NKB]) {
    float mx4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x16& c = sc[i / 2];
      const int r0 = 8 * (i % 2);
      mx4[i] = fmaxf(fmaxf(fmaxf(c[r0], c[r0 + 1]), fmaxf(c[r0 + 2], c[r0 + 3])),
                     fmaxf(fmaxf(c[r0 + 4], c[r0 + 5]), fmaxf(c[r0 + 6], c[r0 + 7])));
    }
    const float mx = max_halves(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]))) * scale2;
    raise = mx > m_run + kRescaleSlack;
    m_new = raise ? fmaxf(m_run, mx) : m_run;
    alpha = (!raise || m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
  };
  // Apply a rescale decision to the running state (before the tile's weights
  // are accumulated).
  auto apply_rescale = [&]() {
    if (__ballot(raise) != 0) {
#pragma unroll
      for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[vb][r] *= alpha;
    }
    l_run *= alpha;
    m_run = m_new;
    neg_m = m_run == -INFINITY ? 0.f : -m_run;
    spec_lim = m_run == -INFINITY ? 0.f : kSpecBound;
  };

  // Dropout draws.  Register r of block kb holds key 32 kb + 8 g + 4 hh + e
  // (g = r / 4, e = r % 4) of the tile for this lane's query: key block
  // k0 / 4 + 8 kb + 2 g + hh, key e in it.  The quad's lanes hold the four
  // queries of one query block, so the quad needs the 8 calls (kb, g) of its
  // half; quad position e' draws calls 2 e' and 2 e' + 1 (counter (key / 4,
  // query / 4, unit, 0)), packed as bit 8 (key % 4) + 4 + query % 4, in the
  // previous step's second phase, where the vector ALUs are otherwise idle.
  // The weights read them across the quad where they are applied.
  uint32_t dc[2][4] = {}, dm[2] = {0u, 0u};
  // A pair's keep mask for the packed bf16 weights comes from one byte
  // permute: shifted left by 11 - query % 4 the call's bits put key 0's flag
  // at bit 15 and key 2's at bit 31, shifted by 3 - query % 4 keys 1 and 3
  // there, and v_perm_b32 replicates the top bit of bytes 1 and 3 of either.
  const uint32_t shx = 11u - (uint32_t)(lane & 3), shy = 3u - (uint32_t)(lane & 3);
  const KeepConsts kq = keep_consts(p.drop.p8);
  auto draw_init = [&](int key0) {  // first key of the tile
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 2 * (lane & 3) + j, kb = c >> 2, g = c & 3;  // call (kb, g) of this lane
      dc[j][0] = ((uint32_t)key0 >> 2) + 8u * (uint32_t)kb + 2u * (uint32_t)g + (uint32_t)hh;
      dc[j][1] = (uint32_t)q >> 2;
      dc[j][2] = (uint32_t)unit;
      dc[j][3] = 0u;
      dm[j] = 0u;
    }
  };
  auto draw_item = [&](int t) {  // call t / 14: rounds 0..9, then the keep bits of its four words
    const int j = t / 14, k = t % 14;
    if (k < 10) philox_round(dc[j][0], dc[j][1], dc[j][2], dc[j][3], p.drop.seed_lo, p.drop.seed_hi, k);
    else dm[j] = pack_keep(dm[j], keep_flags(dc[j][k - 10], kq), k - 10);
  };
  // The draw state is pinned after each slice of items: otherwise the
  // compiler sinks the draws out of the second phase to their first use.
  auto draw_pin = [&]() {
    asm volatile("" : "+v"(dc[0][0]), "+v"(dc[0][1]), "+v"(dc[0][2]), "+v"(dc[0][3]), "+v"(dc[1][0]),
                 "+v"(dc[1][1]), "+v"(dc[1][2]), "+v"(dc[1][3]), "+v"(dm[0]), "+v"(dm[1]));
  };
  auto call_bits = [&](int c) -> uint32_t {  // the keep bits of call c = 4 kb + g of the quad
    const uint32_t x = dm[c & 1];
    switch (c >> 1) {
      case 0: return quad_bcast<0>(x);
      case 1: return quad_bcast<1>(x);
      case 2: return quad_bcast<2>(x);
      default: return quad_bcast<3>(x);
    }
  };
  // Mask of the bf16 pair of registers r, r + 1 (r % 4 in {0, 2}): each half
  // all ones iff its key is kept.
  auto pair_mask = [&](uint32_t bits, int r) -> uint32_t {
    return __builtin_amdgcn_perm(bits << shy, bits << shx, (r & 3) == 0 ? 0x0A0A0808u : 0x0B0B0909u);
  };

  // This split's share of the key tiles [0, kt_end): [t0, kt_end).
  int t0 = 0;
  if (p.splits > 1) {
    const int per = (kt_end + p.splits - 1) / p.splits;
    t0 = split * per < kt_end ? split * per : kt_end;
    kt_end = t0 + per < kt_end ? t0 + per : kt_end;
  }
  if (MASK == kMaskBitmask && t0 < kt_end && tile_class(t0) == kTileEmpty) t0 = next_tile(t0);
  __syncthreads();  // V buffers cleared
  if (t0 < kt_end) {  // workgroup-uniform
    int t1 = next_tile(t0);
    fill_k(t0, kbuf0);
    fill_v(t0, vbuf0);
    if (t1 < kt_end) fill_k(t1, kbuf1);
    wait_vm();
    __syncthreads();
    f32x16 sa[S::NKB], sb[S::NKB];
    if constexpr (DROP) {  // the first tile's calls
      draw_init(t0 * S::BK);
#pragma unroll
      for (int tt = 0; tt < 28; ++tt) draw_item(tt);
    }
    scores(sa, kbuf0);
    if (tile_class(t0) == kTilePartial) mask_tile(sa, t0);
    row_max(sa);
    apply_rescale();
    __syncthreads();  // K buffer 0 free for tile t2

    // One pipeline step.  On entry cur holds the masked S^T of tile t0; nxt
    // receives S^T of tile t1 from knxt.  One scheduling region:
    //   MFMA S^T(t1)             || VALU exp / pack / sums of t0
    //   MFMA O^T += V^T P^T(t0)
    // The weights of t0 are formed against the running reference max before
    // that max is brought up to date (no row max on the common path): a
    // lane whose 32 weights sum to at most 2^(slack - 1) has every score
    // below the reference plus slack - 1, where the lazy-rescale rule keeps
    // the reference.  Otherwise (or for a row that had no allowed key yet)
    // the wave takes the rule's exact path: row max of t0, rescale, and the
    // weights again.  The reference max therefore follows the same rule as
    // with the max computed first.
    auto step = [&](f32x16 (&cur)[S::NKB], f32x16 (&nxt)[S::NKB], char* kcur, char* knxt, char* vcur,
                    char* vnxt) {
      const int t2 = t1 < kt_end ? next_tile(t1) : kt_end;
      // This step's copies (K of t2 into kcur, V of t1 into vnxt) issue one per
      // first-phase MFMA; past the last tile they copy empty ranges.
      const int k2 = t2 < kt_end ? t2 * S::BK : nk, k1 = t1 < kt_end ? t1 * S::BK : nk;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc_rows(Kb + (int64_t)k2 * krow, nk - k2, krow, kmax_rows);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc_rows(Vb + (int64_t)k1 * vrow, nk - k1, vrow, vmax_rows);
      auto copy_item = [&](int i) {
        if (i < S::KWIN) {
          // Every wave has a window for the first KWINS / NW copies: known at
          // compile time, so only the last copy selects its source and target.
          const bool real = S::KWINS % S::NW == 0 || i < S::KWINS / S::NW || w + S::NW * i < S::KWINS;
          dma16(real ? rk : rnone, real ? kcur + (w + S::NW * i) * 1024 : spare, koff[i]);
        } else if (i < S::KWIN + S::VWIN) {
          const int jv = i - S::KWIN;
          const bool real = S::VWINS % S::NW == 0 || jv < S::VWINS / S::NW || w + S::NW * jv < S::VWINS;
          dma16(real ? rv : rnone, real ? vnxt + (w + S::NW * jv) * 1024 : spare, voff[jv]);
        }
      };

      // The instruction order below is the schedule: each micro-step is one
      // MFMA, the LDS reads for a later MFMA, and a slice of VALU work, kept
      // apart by scheduling barriers.
      constexpr int NS = S::NQF * S::NKB;      // score MFMAs
      constexpr int NP = S::NVB * S::BK / 16;  // PV MFMAs
      constexpr int PF = MASK == kMaskBitmask ? 4 : 8;  // K reads in flight (fewer where the mask words need registers)
      constexpr int NPAIR = S::NKB * 8;        // weight pairs of the tile
      auto kread = [&](int i) {  // K fragment of score MFMA i (ks = i / NKB, kb = i % NKB)
        return lds_read_b128(knxt, kbase + 32 * (i % S::NKB) * S::KS + 32 * (i / S::NKB));
      };
      auto vread = [&](int i, int half) {  // V^T fragment half of PV MFMA i (ks = i / NVB, vb = i % NVB)
        const int ks = i / S::NVB, vb = i % S::NVB;
        return lds_read_tr(vcur, vbase + (16 * ks + 8 * half) * S::VS + 64 * vb);
      };

      // ---- phase A: S^T(t1) on the MFMA pipe, weights of t0 on the VALU ----
      // Two waves share each SIMD (one from each workgroup on the CU).  The
      // wave in this phase (MFMAs plus the weights' vector work) takes issue
      // priority over a wave in phase B (MFMAs only), so that the vector work
      // runs beside the other wave's MFMAs.
      __builtin_amdgcn_s_setprio(1);
      u32x4 pk[S::NKB][2];
      float ls[4];
      // Pair pr (registers 2 (pr % 8), +1 of block pr / 8) in two halves,
      // issued one slice apart so that the exponentials' latency is covered:
      // weights_e = the exponentials, weights_f = the sum and the packing.
      float pe[S::NKB * 8][2];
      auto weights_e = [&](int pr, float neg_m) {
        const int kb = pr / 8, r = 2 * (pr % 8);
        pe[pr][0] = fast_exp2(__builtin_fmaf(cur[kb][r], scale2, neg_m));
        pe[pr][1] = fast_exp2(__builtin_fmaf(cur[kb][r + 1], scale2, neg_m));
      };
      auto weights_f = [&](int pr) {
        const int kb = pr / 8, r = 2 * (pr % 8);
        ls[pr % 4] = pr < 4 ? pe[pr][0] + pe[pr][1] : ls[pr % 4] + (pe[pr][0] + pe[pr][1]);
        if constexpr (DROP) {  // the PV product takes the kept weights; L the sum of all
          pk[kb][r / 8][(r / 2) % 4] = pack_bf16x2(pe[pr][0], pe[pr][1]) & pair_mask(call_bits(4 * kb + r / 4), r);
        } else {
          pk[kb][r / 8][(r / 2) % 4] = pack_bf16x2(pe[pr][0], pe[pr][1]);
        }
      };
      auto weights = [&](int pr, float neg_m) {
        weights_e(pr, neg_m);
        weights_f(pr);
      };
      bf16x8 kfr[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) kfr[i] = kread(i);
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb) nxt[kb] = f32x16{};
      i16x4 vfr[4];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        nxt[i % S::NKB] = mfma_bf16(kfr[i % PF], qf[i / S::NKB], nxt[i % S::NKB]);
        if (i + PF < NS) kfr[i % PF] = kread(i + PF);
        copy_item(i);
        if (i == NS - 1) {  // first PV operands
          vfr[0] = vread(0, 0);
          vfr[1] = vread(0, 1);
          vfr[2] = vread(1, 0);
          vfr[3] = vread(1, 1);
        }
        // Slice i: the exponentials of its pairs and the rest of the previous slice's.
#pragma unroll
        for (int k = i * (NPAIR + 1) / NS; k < (i + 1) * (NPAIR + 1) / NS; ++k) {
          if (k < NPAIR) weights_e(k, neg_m);
          if (k > 0) weights_f(k - 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      float lt = (ls[0] + ls[1]) + (ls[2] + ls[3]);
      if (__ballot(lt > spec_lim) != 0) {  // wave-uniform, rare
        row_max(cur);
        if (__ballot(raise) != 0) {
          apply_rescale();
#pragma unroll
          for (int pr = 0; pr < NPAIR; ++pr) weights(pr, neg_m);
          lt = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        }
      }
      l_run += lt;

      __builtin_amdgcn_s_setprio(0);
      // ---- phase B: O^T += V^T P^T(t0) on the MFMA pipe (and t1's draws) ----
      if constexpr (DROP) draw_init(k1);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[(i / S::NVB) / 2][(i / S::NVB) % 2]);
        o[i % S::NVB] = mfma_bf16(join_tr(vfr[2 * (i % 2)], vfr[2 * (i % 2) + 1]), pb, o[i % S::NVB]);
        if (i + 2 < NP) {
          vfr[2 * (i % 2)] = vread(i + 2, 0);
          vfr[2 * (i % 2) + 1] = vread(i + 2, 1);
        }
        if constexpr (DROP) {  // t1's two calls: 28 items over the NP slices
#pragma unroll
          for (int tt = i * 28 / NP; tt < (i + 1) * 28 / NP; ++tt) draw_item(tt);
          draw_pin();
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // else nxt holds scores of stale LDS contents: unused
      if (t1 < kt_end && tile_class(t1) == kTilePartial) mask_tile(nxt, t1);
      wait_vm();
      __syncthreads();
      t0 = t1;
      t1 = t2;
    };
    // Tiles are counted one per step (an atomic only while counting): a
    // loop-carried count costs this kernel 40 registers and spills.
    while (true) {
      step(sa, sb, kbuf0, kbuf1, vbuf0, vbuf1);
      count_tiles(p.tile_count, 1);
      if (t0 >= kt_end) break;
      step(sb, sa, kbuf1, kbuf0, vbuf1, vbuf0);
      count_tiles(p.tile_count, 1);
      if (t0 >= kt_end) break;
    }
  }

  const float l_tot = sum_halves(l_run);
  const float l_norm = l_tot;
  const float inv = l_norm > 0.f ? (DROP ? p.drop.keep_inv : 1.f) / l_norm : 0.f;
  if (p.splits > 1) {  // this split's normalised output and L, for fwd_merge_kernel
    if (qvalid) {
      const int64_t row = ((int64_t)split * p.B * p.H + unit) * n + q;
      float* Op = p.Opart + row * DV;
#pragma unroll
      for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int vd = vb * 32 + 8 * g + 4 * hh;
          *reinterpret_cast<f32x4*>(Op + vd) =
              f32x4{o[vb][4 * g] * inv, o[vb][4 * g + 1] * inv, o[vb][4 * g + 2] * inv, o[vb][4 * g + 3] * inv};
        }
      if (hh == 0)
        p.Lpart[row] = (m_run == -INFINITY || l_tot <= 0.f) ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
    }
    return;
  }
  if (qvalid) {
    const int64_t obase = (int64_t)b * p.so[0] + (int64_t)h * p.so[1] + (int64_t)q * p.so[2];
#pragma unroll
    for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int vd = vb * 32 + 8 * g + 4 * hh;
        const u32x2 pk2{pack_bf16x2(o[vb][4 * g] * inv, o[vb][4 * g + 1] * inv),
                        pack_bf16x2(o[vb][4 * g + 2] * inv, o[vb][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>((char*)p.O + (obase + vd) * 2) = pk2;
      }
    if (hh == 0) {
      const float Lv = (m_run == -INFINITY || l_tot <= 0.f) ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
      p.L[(int64_t)unit * n + q] = Lv;
    }
  }
}

template <bool BF16, int D, int DV, int MASK>
static int launch_one(const FwdParams& p, hipStream_t st) {
  dim3 grid((unsigned)p.grid_pad), block(256);
  if constexpr (BF16 && (D == 64 || D == 128) && (DV == 64 || DV == 128)) {
    if (p.drop.p8 != 0) hipLaunchKernelGGL((fwd_pipe_kernel<D, DV, MASK, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fwd_pipe_kernel<D, DV, MASK, false>), grid, block, 0, st, p);
  } else if (p.drop.p8 != 0) {
    hipLaunchKernelGGL((fwd_kernel<BF16, D, DV, MASK, true>), grid, block, 0, st, p);
  } else {
    hipLaunchKernelGGL((fwd_kernel<BF16, D, DV, MASK>), grid, block, 0, st, p);
  }
  return (int)hipGetLastError();
}

template <bool BF16, int D, int DV>
static int launch_mask(const FwdParams& p, int mask_mode, hipStream_t st) {
  switch (mask_mode) {
    case kMaskNone: return launch_one<BF16, D, DV, kMaskNone>(p, st);
    case kMaskCausal: return launch_one<BF16, D, DV, kMaskCausal>(p, st);
    default: return launch_one<BF16, D, DV, kMaskBitmask>(p, st);
  }
}

template <bool BF16>
static int launch_dims(const FwdParams& p, int d, int v, int mask_mode, hipStream_t st) {
  if (d == 64 && v == 64) return launch_mask<BF16, 64, 64>(p, mask_mode, st);
  if (d == 80 && v == 80) return launch_mask<BF16, 80, 80>(p, mask_mode, st);
  if (d == 128 && v == 128) return launch_mask<BF16, 128, 128>(p, mask_mode, st);
  if (d == 64 && v == 128) return launch_mask<BF16, 64, 128>(p, mask_mode, st);
  return (int)hipErrorInvalidValue;
}

// Merge of the split forward's partial results: L = ln sum_s e^{L_s} and
// O = sum_s e^{L_s - L} O_s (the merge of row summaries in its L form; a
// split with no allowed key for the row has L_s = -inf and weight 0).  One
// thread per (row, 4 output columns).
template <bool BF16, int DV>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p) {
  const int64_t rows = (int64_t)p.B * p.H * p.n;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (DV / 4)) return;
  const int64_t row = t / (DV / 4);
  const int c4 = (int)(t % (DV / 4));
  float mx = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.Lpart[s * rows + row]);
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int s = 0; s < p.splits; ++s) sum += expf(p.Lpart[s * rows + row] - mx);
    L = mx + logf(sum);
    for (int s = 0; s < p.splits; ++s) {
      const float ws = expf(p.Lpart[s * rows + row] - L);
      const f32x4 x = *reinterpret_cast<const f32x4*>(p.Opart + (s * rows + row) * DV + 4 * c4);
      acc += f32x4{ws * x[0], ws * x[1], ws * x[2], ws * x[3]};
    }
  }
  const int64_t unit = row / p.n, i = row % p.n;
  const int64_t b = unit / p.H, h = unit % p.H;
  const int64_t off = b * p.so[0] + h * p.so[1] + i * p.so[2] + 4 * c4;
  if constexpr (BF16)
    *reinterpret_cast<u32x2*>((char*)p.O + off * 2) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  else
    *reinterpret_cast<f32x4*>((char*)p.O + off * 4) = acc;
  if (c4 == 0) p.L[row] = L;
}

int launch_fwd_merge(const FwdParams& p, int bf16, int v, void* stream) {
  const int64_t threads = (int64_t)p.B * p.H * p.n * (v / 4);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  hipStream_t st = (hipStream_t)stream;
  if (!bf16) return (int)hipErrorInvalidValue;  // splitting is a bf16-only path
  if (v == 64) hipLaunchKernelGGL((fwd_merge_kernel<true, 64>), grid, block, 0, st, p);
  else if (v == 128) hipLaunchKernelGGL((fwd_merge_kernel<true, 128>), grid, block, 0, st, p);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_fwd(const FwdParams& p, int bf16, int d, int v, int mask_mode, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return bf16 ? launch_dims<true>(p, d, v, mask_mode, st) : launch_dims<false>(p, d, v, mask_mode, st);
}

}  // namespace eta
