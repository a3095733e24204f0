// Backward, query-tile-outer dQ kernel.
//
// Method (alphabetamath page, reverse procedure; ob1 page, part 2;
// HarshvardhanJ README, backward section): with the forward's L and
// D_i = <dO_i, O_i>, for every allowed (i, j) recompute s_ij = c <Q_i, K_j>,
// p_ij = exp(s_ij - L_i), dS_ij = p_ij (<dO_i, V_j> - D_i) and accumulate
// dQ_i += c dS_ij K_j.  Each workgroup owns 128 query rows and streams the
// key tiles, so every dQ row is summed by one lane in a fixed order: the
// result is deterministic and needs no atomics.
//
// gfx950 design, the same shape as the forward kernel: one lane per query
// column.  S^T = K Q^T and dP^T = V dO^T on MFMA with the wave's Q and dO
// rows held in registers as B operands and the K and V tiles read from LDS
// as row operands; L_i and D_i are per-lane scalars; dS^T stays in the
// score registers and is the B operand of dQ^T += K^T dS^T, whose K^T
// operand comes from the same K tile through transposed reads (the K tile
// is read both ways).  K and V tiles of 64 keys are double-buffered through
// XOR-swizzled LDS; two workgroups share a CU.
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {

template <bool BF16, int D, int DV>
struct DqShape {
  static constexpr int NW = 4;
  static constexpr int BQ = kDqBq;
  static constexpr int BK = kDqBk;
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int KSTEP = BF16 ? 16 : 2;
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  static constexpr int NKB = BK / 32;
  static constexpr int KCH = D * ES / 16;   // loaded 16-byte chunks per K row
  static constexpr int VCH = DV * ES / 16;  // loaded 16-byte chunks per V row
  using KT = Swz<DP * ES / 16>;             // K tile (padded to DP columns for the transposed reads)
  using VT = Swz<VCH>;
  static constexpr int KTILE = BK * KT::kStride;
  static constexpr int VTILE = BK * VT::kStride;
  static constexpr int KLD = (BK * KCH + 255) / 256;
  static constexpr int VLD = (BK * VCH + 255) / 256;
  static constexpr int NQF = D / KSTEP;
  static constexpr int NOF = DV / KSTEP;
  static constexpr int SMEM = 2 * (KTILE + VTILE);
};

// DROP: dS = P ((dO V^T) o Z / keep - D) with the replayed keep decisions.
template <bool BF16, int D, int DV, int MASK, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BF16 ? 2 : 1, 2))) void bwd_dq_kernel(BwdParams p) {
  using S = DqShape<BF16, D, DV>;
  __shared__ __attribute__((aligned(16))) char smem[S::SMEM];

  const int64_t logical = xcd_logical(blockIdx.x, p.grid_pad_dq, p.total_dq);
  if (logical < 0) return;
  const int unit = (int)(logical / p.tq_dq);
  const int qt = p.tq_dq - 1 - (int)(logical % p.tq_dq);  // heaviest causal tiles first
  const int b = unit / p.H, h = unit % p.H;
  const int n = (int)p.n, nk = (int)p.nk, coff = (int)p.coff;  // query rows, key rows, causal offset
  const int q0 = qt * S::BQ;
  const int tk = (nk + S::BK - 1) / S::BK;

  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int hh = lane >> 5;
  const int g1 = (lane >> 4) & 1;
  const int q = q0 + 32 * w + (lane & 31);
  const bool qvalid = q < n;

  const int qrow = (int)p.sq[2] * S::ES, krow = (int)p.sk[2] * S::ES;
  const int vrow = (int)p.sv[2] * S::ES, orow = (int)p.so[2] * S::ES;
  const char* Qb = (const char*)p.Q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]) * S::ES;
  const char* Kb = (const char*)p.K + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]) * S::ES;
  const char* Vb = (const char*)p.V + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]) * S::ES;
  const char* dOb = (const char*)p.dO + ((int64_t)b * p.so[0] + (int64_t)h * p.so[1]) * S::ES;

  // Per-lane row statistics.  Rows with L = -inf (no allowed key) or past n
  // use +inf, so that p = exp2(s - inf) = 0.
  float L2 = INFINITY, Dq = 0.f;
  if (qvalid) {
    const float Lv = p.L[(int64_t)unit * n + q];
    L2 = (Lv == -INFINITY) ? INFINITY : Lv * kLog2e;
    Dq = -p.Dn[(int64_t)unit * p.n_pad + q];
  }

  // Q and dO rows as B operands.
  typedef typename std::conditional<BF16, bf16x8, float>::type Frag;
  Frag qf[S::NQF], of[S::NOF];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb, (int64_t)n * qrow);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(dOb, (int64_t)n * orow);
#pragma unroll
    for (int s = 0; s < S::NQF; ++s) {
      if constexpr (BF16)
        qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, q * qrow + (16 * s + 8 * hh) * 2, 0, 0));
      else
        qf[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rq, q * qrow + (2 * s + hh) * 4, 0, 0));
    }
#pragma unroll
    for (int s = 0; s < S::NOF; ++s) {
      if constexpr (BF16)
        of[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, q * orow + (16 * s + 8 * hh) * 2, 0, 0));
      else
        of[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ro, q * orow + (2 * s + hh) * 4, 0, 0));
    }
  }

  int kt_end = tk;
  if constexpr (MASK == kMaskCausal) {
    const int k_hi = (q0 + S::BQ < n ? q0 + S::BQ : n) - 1 + coff;  // last key any row allows
    kt_end = k_hi < 0 ? 0 : (k_hi / S::BK + 1 < tk ? k_hi / S::BK + 1 : tk);
  }
  const uint8_t* map_row = nullptr;
  const uint32_t* mrow = nullptr;
  if constexpr (MASK == kMaskBitmask) {
    const int64_t mu = p.mask_sb == 0 ? h : unit;
    map_row = p.map_dq + (mu * p.tq_dq + qt) * (int64_t)tk;
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

  // Zero the padded K columns of both buffers once (only when D % 32).
  if constexpr (S::DP != D) {
    constexpr int padc = (S::DP - D) * S::ES / 16;
    for (int c = tid; c < 2 * S::BK * padc; c += 256) {
      const int bf = c / (S::BK * padc), r = (c / padc) % S::BK, cc = c % padc;
      *reinterpret_cast<u32x4*>(smem + bf * (S::KTILE + S::VTILE) + S::KT::off(r, S::KCH + cc)) = u32x4{0, 0, 0, 0};
    }
  }

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

  f32x16 dq[S::NDB];
#pragma unroll
  for (int i = 0; i < S::NDB; ++i) dq[i] = f32x16{};

  int kt = 0;
  if (MASK == kMaskBitmask && kt < kt_end && tile_class(kt) == kTileEmpty) kt = next_tile(kt);
  if (kt < kt_end) {
    gload(kt);
    lstore(0);
  }
  __syncthreads();
  int buf = 0, ntiles = 0;
  const int wave_k_hi = q0 + 32 * w + 31 + coff;  // last key this wave's rows can allow
  const float scale2 = p.scale2;

  while (kt < kt_end) {
    const int kn = next_tile(kt);
    const uint8_t cls = tile_class(kt);
    if (kn < kt_end) gload(kn);
    const int k0 = kt * S::BK;
    const char* Ks = smem + buf * (S::KTILE + S::VTILE);
    const char* Vs = Ks + S::KTILE;

    bool active = true;
    if constexpr (MASK == kMaskCausal) active = k0 <= wave_k_hi;
    if (active) {
      f32x16 s[S::NKB], dp[S::NKB];
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < S::NQF; ++ks)
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb) {
          if constexpr (BF16)
            s[kb] = mfma_bf16(lds_read_b128(Ks, S::KT::off(32 * kb + (lane & 31), 2 * ks + hh)), qf[ks], s[kb]);
          else
            s[kb] = mfma_f32(*reinterpret_cast<const float*>(Ks + S::KT::off_dword(32 * kb + (lane & 31), 2 * ks + hh)),
                             qf[ks], s[kb]);
        }
#pragma unroll
      for (int ks = 0; ks < S::NOF; ++ks)
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb) {
          if constexpr (BF16)
            dp[kb] = mfma_bf16(lds_read_b128(Vs, S::VT::off(32 * kb + (lane & 31), 2 * ks + hh)), of[ks], dp[kb]);
          else
            dp[kb] = mfma_f32(*reinterpret_cast<const float*>(Vs + S::VT::off_dword(32 * kb + (lane & 31), 2 * ks + hh)),
                              of[ks], dp[kb]);
        }
      // dS = P (dP - D), P = exp2(s c log2 e - L log2 e); register r of block
      // kb holds key 32 kb + 8 (r/4) + 4 hh + r%4 of the tile.
      u32x4 pk[S::NKB][2];
#pragma unroll
      for (int kb = 0; kb < S::NKB; ++kb) {
        uint32_t word = 0xFFFFFFFFu;
        if constexpr (MASK == kMaskBitmask) {
          if (cls == kTilePartial && qvalid && k0 + 32 * kb < nk) word = mrow[(k0 + 32 * kb) >> 5];
        }
        // Dropout: registers 4g..4g+3 hold 4 consecutive keys of this lane's
        // row; the quad's lanes hold rows 4a..4a+3 (see the forward).
        uint32_t keepg[4] = {0xFu, 0xFu, 0xFu, 0xFu};
        if constexpr (DROP) {
          const uint32_t e = (uint32_t)lane & 3u;
          const uint32_t m = keep_mask16(p.drop.seed_lo, p.drop.seed_hi, p.drop.p8,
                                         (uint32_t)(k0 + 32 * kb + 8 * (int)e + 4 * hh) >> 2, (uint32_t)q >> 2,
                                         (uint32_t)unit, false);
          keepg[0] = (quad_bcast<0>(m) >> (4 * e)) & 0xFu;
          keepg[1] = (quad_bcast<1>(m) >> (4 * e)) & 0xFu;
          keepg[2] = (quad_bcast<2>(m) >> (4 * e)) & 0xFu;
          keepg[3] = (quad_bcast<3>(m) >> (4 * e)) & 0xFu;
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const uint32_t keep = keepg[r >> 2];
          float ds[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float pv = fast_exp2(__builtin_fmaf(s[kb][r + e], scale2, -L2));
            if (cls == kTilePartial) {
              const int kk = 32 * kb + 8 * ((r + e) >> 2) + 4 * hh + ((r + e) & 3);
              const int key = k0 + kk;
              bool ok = key < nk;
              if constexpr (MASK == kMaskCausal) ok = ok && key <= q + coff;
              if constexpr (MASK == kMaskBitmask) ok = ok && ((word >> (kk & 31)) & 1u);
              pv = ok ? pv : 0.f;
            }
            if constexpr (DROP) {
              const bool z = (keep >> ((r + e) & 3)) & 1u;
              ds[e] = pv * ((z ? dp[kb][r + e] : 0.f) - Dq) * p.drop.keep_inv;  // Dq = D P(keep)
            } else {
              ds[e] = pv * (dp[kb][r + e] - Dq);
            }
          }
          if constexpr (BF16)
            pk[kb][r / 8][(r / 2) % 4] = pack_bf16x2(ds[0], ds[1]);
          else {
            s[kb][r] = ds[0];
            s[kb][r + 1] = ds[1];
          }
        }
      }
      // dQ^T += K^T dS^T.
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < S::BK / 16; ++ks) {
          const bf16x8 sb = __builtin_bit_cast(bf16x8, pk[ks / 2][ks % 2]);
#pragma unroll
          for (int db = 0; db < S::NDB; ++db) {
            const int n0 = db * 32 + 16 * g1;
            const i16x4 lo = lds_read_tr(Ks, S::KT::tr(lane, 16 * ks + 4 * hh, n0));
            const i16x4 hi = lds_read_tr(Ks, S::KT::tr(lane, 16 * ks + 8 + 4 * hh, n0));
            dq[db] = mfma_bf16(join_tr(lo, hi), sb, dq[db]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
              const float a = *reinterpret_cast<const float*>(Ks + S::KT::off_dword(kk, db * 32 + (lane & 31)));
              dq[db] = mfma_f32(a, s[kb][r], dq[db]);
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
  count_tiles(p.tile_count_dq, ntiles);

  // dQ = c dQ^T (lane = query row; 4 consecutive columns per store).
  if (qvalid) {
    char* dQp = (char*)p.dQ + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1] + (int64_t)q * p.sq[2]) * S::ES;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = db * 32 + 8 * g + 4 * hh;
        if (c0 < D) {
          const float x0 = dq[db][4 * g] * p.scale, x1 = dq[db][4 * g + 1] * p.scale;
          const float x2 = dq[db][4 * g + 2] * p.scale, x3 = dq[db][4 * g + 3] * p.scale;
          if constexpr (BF16)
            *reinterpret_cast<u32x2*>(dQp + c0 * 2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          else
            *reinterpret_cast<f32x4*>(dQp + c0 * 4) = f32x4{x0, x1, x2, x3};
        }
      }
  }
}

template <bool BF16, int D, int DV, int MASK>
static int launch_one(const BwdParams& p, hipStream_t st) {
  if (p.drop.p8 != 0)
    hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, DV, MASK, true>), dim3((unsigned)p.grid_pad_dq), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, DV, MASK>), dim3((unsigned)p.grid_pad_dq), dim3(256), 0, st, p);
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

int launch_bwd_dq(const BwdParams& p, int bf16, int d, int v, int mask_mode, void* stream) {
  if (bwd_dq_pipe_supported(bf16, d, v, mask_mode, p.nk))
    return launch_bwd_dq_pipe(p, d, v, mask_mode, stream);
  hipStream_t st = (hipStream_t)stream;
  return bf16 ? launch_dims<true>(p, d, v, mask_mode, st) : launch_dims<false>(p, d, v, mask_mode, st);
}

}  // namespace eta
