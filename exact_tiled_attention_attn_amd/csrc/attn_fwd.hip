// Forward kernel: exact attention with an online softmax over key tiles.
//
// Method (ob1 page, part 1; trentorch exercise, hint and constraints;
// maitreyasuin post, the tiled forward): per query row keep the running
// maximum m, the running denominator l and the unnormalised output; for each
// key tile take m' = max(m, tile max), rescale l and the output by
// exp(m - m'), add exp(s - m') and its product with V; normalise once at the
// end and keep L = m + ln l.  Tiles whose intersection with every row's
// allowed set is empty are skipped and only partially allowed tiles are
// masked (ob1 page, part 3; alphabetamath page, forward step 2).
//
// gfx950 design.  One workgroup = 4 waves = 128 query rows; each wave owns
// 32 rows.  Scores are formed transposed, S^T = K Q^T, with the wave's Q
// rows held in registers as the MFMA B operand, so every lane owns one
// query column: the row max and row sum are in-lane reductions plus one
// permlane32 swap between the two half-waves, and the rescale factor is a
// per-lane scalar.  The output accumulator is kept transposed too,
// O^T += V^T P^T, with P^T fed from the score registers (converted to bf16)
// and V^T read from the row-major V tile in LDS with transposed reads
// (ds_read_b64_tr_b16); the order in which a lane holds its keys is matched
// by the read addresses, so no shuffle is needed.  K and V tiles of 64 keys
// are staged through two LDS buffers: the next tile's global loads are in
// flight while the current tile is computed.  Scores use the base-2
// exponential with c log2(e) folded into the scale.
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
  static constexpr int KSTR = D * ES + 16;                  // bytes per K row in LDS
  static constexpr int VSTR = DVP * ES + 16;                // bytes per V row in LDS
  static constexpr int KTILE = BK * KSTR;
  static constexpr int VTILE = BK * VSTR;
  static constexpr int KCH = D * ES / 16;   // 16-byte chunks per K row
  static constexpr int VCH = DV * ES / 16;  // 16-byte chunks per V row
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

template <bool BF16, int D, int DV, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(FwdParams p) {
  using S = FwdShape<BF16, D, DV>;
  __shared__ __attribute__((aligned(16))) char smem[S::SMEM];

  const int64_t logical = xcd_logical(blockIdx.x, p.grid_pad, p.total);
  if (logical < 0) return;
  const int64_t unit = logical / p.tq;
  const int qt = p.tq - 1 - (int)(logical % p.tq);  // heaviest causal tiles first
  const int b = (int)(unit / p.H), h = (int)(unit % p.H);
  const int64_t n = p.n;
  const int64_t q0 = (int64_t)qt * S::BQ;

  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int hh = lane / 32;  // half-wave
  const int64_t q = q0 + 32 * w + (lane & 31);
  const bool qvalid = q < n;

  const char* Qb = (const char*)p.Q + (b * p.sq[0] + h * p.sq[1]) * S::ES;
  const char* Kb = (const char*)p.K + (b * p.sk[0] + h * p.sk[1]) * S::ES;
  const char* Vb = (const char*)p.V + (b * p.sv[0] + h * p.sv[1]) * S::ES;

  // Q fragments (B operand of S^T = K Q^T).  For c < 0 the rows are negated
  // (exact) and |c| is used, so the tile max is taken on raw scores.
  // |c| log2(e) is clamped to >= 1e-30: for c = 0 every score then maps to
  // exp2(~1e-24) = 1.0f exactly, while masked scores (-inf) stay -inf.
  const bool neg = p.scale2 < 0.f;
  const float scale2 = fmaxf(fabsf(p.scale2), 1e-30f);
  typedef typename std::conditional<BF16, bf16x8, float>::type QFrag;
  QFrag qf[S::NQF];
#pragma unroll
  for (int ks = 0; ks < S::NQF; ++ks) {
    if constexpr (BF16) {
      u32x4 x = qvalid ? *reinterpret_cast<const u32x4*>(Qb + (q * p.sq[2] + 16 * ks + 8 * hh) * 2)
                       : u32x4{0, 0, 0, 0};
      if (neg) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[ks] = *reinterpret_cast<bf16x8*>(&x);
    } else {
      const float x = qvalid ? *reinterpret_cast<const float*>(Qb + (q * p.sq[2] + 2 * ks + hh) * 4) : 0.f;
      qf[ks] = neg ? -x : x;
    }
  }

  // Key-tile range and classification.
  int kt_end = p.tk;
  if constexpr (MASK == kMaskCausal) {
    int64_t q_hi = (q0 + S::BQ < n ? q0 + S::BQ : n) - 1;
    kt_end = (int)(q_hi / S::BK) + 1;
  }
  const uint8_t* map_row = nullptr;
  const uint32_t* mrow = nullptr;
  if constexpr (MASK == kMaskBitmask) {
    int64_t mu = p.mask_sb == 0 ? h : unit;
    map_row = p.map + (mu * p.tq + qt) * (int64_t)p.tk;
    mrow = p.mask + b * p.mask_sb + h * p.mask_sh + (qvalid ? q : 0) * p.mask_si;
  }
  auto tile_class = [&](int kt) -> uint8_t {
    if constexpr (MASK == kMaskBitmask) return map_row[kt];
    return classify_analytic(MASK, q0, S::BQ, (int64_t)kt * S::BK, S::BK, n);
  };
  auto next_tile = [&](int kt) -> int {
    for (int k = kt + 1; k < kt_end; ++k)
      if (tile_class(k) != kTileEmpty) return k;
    return kt_end;
  };

  // Zero the padded value columns of both V buffers once (only when DV % 32).
  if constexpr (S::DVP != DV) {
    constexpr int padc = (S::DVP - DV) * S::ES / 16;
    for (int c = tid; c < 2 * S::BK * padc; c += 256) {
      int buf = c / (S::BK * padc), r = (c / padc) % S::BK, cc = c % padc;
      *reinterpret_cast<u32x4*>(smem + buf * (S::KTILE + S::VTILE) + S::KTILE + r * S::VSTR +
                                DV * S::ES + cc * 16) = u32x4{0, 0, 0, 0};
    }
  }

  u32x4 kreg[S::KLD], vreg[S::VLD];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * S::BK;
#pragma unroll
    for (int i = 0; i < S::KLD; ++i) {
      int c = tid + i * 256;
      int r = c / S::KCH, cc = c % S::KCH;
      int64_t key = k0 + r;
      kreg[i] = (c < S::BK * S::KCH && key < n)
                    ? *reinterpret_cast<const u32x4*>(Kb + key * p.sk[2] * S::ES + cc * 16)
                    : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < S::VLD; ++i) {
      int c = tid + i * 256;
      int r = c / S::VCH, cc = c % S::VCH;
      int64_t key = k0 + r;
      vreg[i] = (c < S::BK * S::VCH && key < n)
                    ? *reinterpret_cast<const u32x4*>(Vb + key * p.sv[2] * S::ES + cc * 16)
                    : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
    char* kt_s = smem + buf * (S::KTILE + S::VTILE);
    char* vt_s = kt_s + S::KTILE;
#pragma unroll
    for (int i = 0; i < S::KLD; ++i) {
      int c = tid + i * 256;
      if (c < S::BK * S::KCH)
        *reinterpret_cast<u32x4*>(kt_s + (c / S::KCH) * S::KSTR + (c % S::KCH) * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < S::VLD; ++i) {
      int c = tid + i * 256;
      if (c < S::BK * S::VCH)
        *reinterpret_cast<u32x4*>(vt_s + (c / S::VCH) * S::VSTR + (c % S::VCH) * 16) = vreg[i];
    }
  };

  // Running state for this lane's query row (both half-waves hold it).
  float m_run = -INFINITY;
  // This half-wave's partial denominators: l_run sums the fp32 weights (for
  // L); l_use sums the weights as the PV product consumes them (bf16-rounded
  // on the bf16 path), so that O is normalised by the weights actually used.
  float l_run = 0.f, l_use = 0.f;
  f32x16 o[S::NVB];
#pragma unroll
  for (int vb = 0; vb < S::NVB; ++vb) o[vb] = f32x16{};

  int kt = next_tile(-1);
  if (kt < kt_end) {
    gload(kt);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  const int64_t wave_q_hi = q0 + 32 * w + 31;

  while (kt < kt_end) {
    const int nk = next_tile(kt);
    const uint8_t cls = tile_class(kt);
    if (nk < kt_end) gload(nk);
    const int64_t k0 = (int64_t)kt * S::BK;
    const char* Ks = smem + buf * (S::KTILE + S::VTILE);
    const char* Vs = Ks + S::KTILE;

    bool active = true;
    if constexpr (MASK == kMaskCausal) active = k0 <= wave_q_hi;  // wave-uniform
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
            bf16x8 a = lds_read_b128(Ks, (32 * kb + (lane & 31)) * S::KSTR + (16 * ks + 8 * hh) * 2);
            s[kb] = mfma_bf16(a, qf[ks], s[kb]);
          } else {
            float a = *reinterpret_cast<const float*>(Ks + (32 * kb + (lane & 31)) * S::KSTR +
                                                      (2 * ks + hh) * 4);
            s[kb] = mfma_f32(a, qf[ks], s[kb]);
          }
        }
      }
      // Mask partial tiles; tile row max on raw scores (scale2 >= 0).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb) {
        uint32_t word = 0xFFFFFFFFu;
        if constexpr (MASK == kMaskBitmask) {
          if (cls == kTilePartial && qvalid && k0 + 32 * kb < n) word = mrow[(k0 + 32 * kb) >> 5];
        }
        if (cls == kTilePartial) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int64_t key = k0 + kk;
            bool ok = key < n;
            if constexpr (MASK == kMaskCausal) ok = ok && key <= q;
            if constexpr (MASK == kMaskBitmask) ok = ok && ((word >> (kk & 31)) & 1u);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = max_halves(mx) * scale2;  // base-2 units; -inf stays -inf (scale2 > 0)
      // Raise the reference max only when it is exceeded by more than the
      // slack (wave-uniform decision).
      if (__ballot(mx > m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
        l_use *= alpha;
#pragma unroll
        for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[vb][r] *= alpha;
        m_run = m_new;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      uint32_t pk[S::NKB][8];  // bf16 path: weights packed in pairs for the PV MFMA
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], scale2, neg_m));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], scale2, neg_m));
          l_run += p0 + p1;
          if constexpr (BF16) {
            const uint32_t u = pack_bf16x2(p0, p1);
            pk[kb][r / 2] = u;
            l_use = __builtin_amdgcn_fdot2_f32_bf16(*reinterpret_cast<const bf16x2*>(&u), ones_bf16x2(), l_use, false);
          } else {
            s[kb][r] = p0;
            s[kb][r + 1] = p1;
          }
        }
      if constexpr (!BF16) l_use = l_run;

      // O^T += V^T P^T.
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < S::BK / 16; ++ks) {
          const u32x4 pw{pk[ks / 2][4 * (ks % 2)], pk[ks / 2][4 * (ks % 2) + 1],
                         pk[ks / 2][4 * (ks % 2) + 2], pk[ks / 2][4 * (ks % 2) + 3]};
          const bf16x8 pb = *reinterpret_cast<const bf16x8*>(&pw);
          const int g1 = (lane >> 4) & 1;
#pragma unroll
          for (int vb = 0; vb < S::NVB; ++vb) {
            const int n0 = vb * 32 + 16 * g1;
            i16x4 lo = lds_read_tr(Vs, tr_addr(lane, 16 * ks + 4 * hh, n0, S::VSTR));
            i16x4 hi = lds_read_tr(Vs, tr_addr(lane, 16 * ks + 8 + 4 * hh, n0, S::VSTR));
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
              float a = *reinterpret_cast<const float*>(Vs + kk * S::VSTR + (vb * 32 + (lane & 31)) * 4);
              o[vb] = mfma_f32(a, s[kb][r], o[vb]);
            }
          }
      }
    }
    if (nk < kt_end) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    kt = nk;
  }

  // Epilogue: O = acc / l, L = (m + log2 l) ln 2.
  const float l_tot = sum_halves(l_run);
  const float l_norm = sum_halves(l_use);
  const float inv = l_norm > 0.f ? 1.f / l_norm : 0.f;
  if (qvalid) {
    const int64_t obase = b * p.so[0] + h * p.so[1] + q * p.so[2];
#pragma unroll
    for (int vb = 0; vb < S::NVB; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int vd = vb * 32 + 8 * g + 4 * hh;
        if (vd < DV) {
          float x0 = o[vb][4 * g] * inv, x1 = o[vb][4 * g + 1] * inv;
          float x2 = o[vb][4 * g + 2] * inv, x3 = o[vb][4 * g + 3] * inv;
          if constexpr (BF16) {
            u32x2 pk{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
            *reinterpret_cast<u32x2*>((char*)p.O + (obase + vd) * 2) = pk;
          } else {
            *reinterpret_cast<f32x4*>((char*)p.O + (obase + vd) * 4) = f32x4{x0, x1, x2, x3};
          }
        }
      }
    if (hh == 0) {
      const float Lv = (m_run == -INFINITY || l_tot <= 0.f) ? -INFINITY
                                                             : (m_run + fast_log2(l_tot)) * kLn2;
      p.L[unit * n + q] = Lv;
    }
  }
}

template <bool BF16, int D, int DV, int MASK>
static int launch_one(const FwdParams& p, hipStream_t st) {
  dim3 grid((unsigned)p.grid_pad), block(256);
  hipLaunchKernelGGL((fwd_kernel<BF16, D, DV, MASK>), grid, block, 0, st, p);
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

int launch_fwd(const FwdParams& p, int bf16, int d, int v, int mask_mode, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return bf16 ? launch_dims<true>(p, d, v, mask_mode, st) : launch_dims<false>(p, d, v, mask_mode, st);
}

}  // namespace eta
