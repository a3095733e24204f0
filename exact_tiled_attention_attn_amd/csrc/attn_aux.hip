// Memory-bound helper kernels of the attention path.
//
// * tile_map_kernel: classifies every (query tile, key tile) pair of an
//   explicit allowed-key bitmask as empty (skipped), partial (masked inside)
//   or full, so that the compute kernels skip blocks with no allowed key
//   (alphabetamath page, forward step 2) and mask only partial ones (ob1
//   page, part 3).  Integer OR/AND over the mask words: HBM-bound.
// * bwd_pre_kernel: D_i = <dO_i, O_i> in fp32 (HarshvardhanJ README,
//   backward section: D costs O(n d) and replaces a pass over P; ob1 page,
//   part 2), L_i log2(e) for the base-2 exponentials of the backward (and
//   -L_i log2(e) / (c log2(e)) for the kernel whose score products start
//   from it), and, on the atomic path, clears the fp32 dQ accumulator.
// * bwd_post_kernel: dQ = c * accumulator, converted to the output type.
#include "../../include/attn.h"
#include "attn_internal.h"
#include "kern_common.h"

namespace eta {

__global__ __launch_bounds__(256) void tile_map_kernel(MapParams p) {
  const int mu = blockIdx.x / p.tq;
  const int a = blockIdx.x % p.tq;
  const int64_t n = p.n, nk = p.nk;  // query rows, key rows
  const int64_t q0 = (int64_t)a * p.bq;
  const int64_t q1 = (q0 + p.bq < n) ? q0 + p.bq : n;
  uint8_t* out = p.map + ((int64_t)mu * p.tq + a) * p.tk;
  if (p.mask_mode != kMaskBitmask) {
    for (int kt = threadIdx.x; kt < p.tk; kt += blockDim.x)
      out[kt] = classify_analytic(p.mask_mode, q0, p.bq, (int64_t)kt * p.bk, p.bk, n, nk, p.coff);
    return;
  }
  int64_t base;
  if (p.units == p.H) {
    base = (int64_t)mu * p.mask_sh;  // mask shared across the batch
  } else {
    base = (int64_t)(mu / p.H) * p.mask_sb + (int64_t)(mu % p.H) * p.mask_sh;
  }
  const int64_t W = (nk + 31) / 32;
  const uint32_t tail_bits = (nk % 32) ? ((1u << (nk % 32)) - 1u) : 0xFFFFFFFFu;
  const int wpt = p.bk / 32;  // words per key tile
  // 64 key tiles per pass, each shared by four row groups (rows q0 + g,
  // q0 + g + 4, ...); the groups' any / all are combined through LDS.
  constexpr int kGroups = 4;
  __shared__ uint32_t s_any[kGroups][64];
  __shared__ uint32_t s_all[kGroups][64];
  const int col = threadIdx.x & 63, g = threadIdx.x >> 6;
  for (int k0 = 0; k0 < p.tk; k0 += 64) {  // uniform trip count: every thread reaches the barriers
    const int kt = k0 + col;
    uint32_t any = 0;
    bool all = (int64_t)(kt + 1) * p.bk <= nk;
    if (kt < p.tk) {
      for (int64_t r = q0 + g; r < q1; r += kGroups) {
        const uint32_t* row = p.mask + base + r * p.mask_si;
        for (int wi = 0; wi < wpt; ++wi) {
          const int64_t wd = (int64_t)kt * wpt + wi;
          if (wd < W) {
            const uint32_t valid = (wd == W - 1) ? tail_bits : 0xFFFFFFFFu;
            const uint32_t x = row[wd] & valid;
            any |= x;
            all = all && (x == valid);
          }
        }
      }
    }
    s_any[g][col] = any;
    s_all[g][col] = all ? 1u : 0u;
    __syncthreads();
    if (g == 0 && kt < p.tk) {
      const uint32_t an = s_any[0][col] | s_any[1][col] | s_any[2][col] | s_any[3][col];
      const uint32_t al = s_all[0][col] & s_all[1][col] & s_all[2][col] & s_all[3][col];
      out[kt] = an ? (al ? kTileFull : kTilePartial) : kTileEmpty;
    }
    __syncthreads();
  }
}

int launch_tile_map(const MapParams& p, void* stream) {
  const int64_t blocks = (int64_t)p.units * p.tq;
  if (blocks <= 0) return 0;
  hipLaunchKernelGGL(tile_map_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------

template <bool BF16, int DV>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int64_t zero_n4) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VCH = DV * ES / 16;  // 16-byte chunks per row
  const int64_t rows = (int64_t)p.B * p.H * p.n_pad;
  const int64_t row = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
  const int sub = threadIdx.x % 16;
  const int64_t unit = row / p.n_pad, i = row % p.n_pad;
  float acc = 0.f;
  if (row < rows && i < p.n) {
    const int64_t b = unit / p.H, h = unit % p.H;
    const int64_t off = (b * p.so[0] + h * p.so[1] + i * p.so[2]) * ES;
    const char* Op = (const char*)p.O + off;
    const char* Gp = (const char*)p.dO + off;
    for (int c = sub; c < VCH; c += 16) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(Op + c * 16);
      const u32x4 g = *reinterpret_cast<const u32x4*>(Gp + c * 16);
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += bf16_bits_to_f32(x[e] & 0xFFFFu) * bf16_bits_to_f32(g[e] & 0xFFFFu);
          acc += bf16_bits_to_f32(x[e] >> 16) * bf16_bits_to_f32(g[e] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += __uint_as_float(x[e]) * __uint_as_float(g[e]);
      }
    }
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (row < rows && sub == 0) {
    // Padding rows (i >= n): D = 0 and L2 = +inf, i.e. zero weights.
    float l2 = INFINITY;
    if (i < p.n) {
      const float Lv = p.L[unit * p.n + i];
      l2 = Lv == -INFINITY ? INFINITY : Lv * kLog2e;
    }
    // With dropout -D P(keep): the dropout kernels start dP from it and
    // apply 1 / P(keep) at the end (P(keep) = 1 - p8 / 256, exact in fp32).
    p.Dn[row] = -acc * ((float)(256u - p.drop.p8) * (1.f / 256.f));
    p.L2[row] = l2;
    if (p.Ls != nullptr) p.Ls[row] = -l2 / (p.scale2 == 0.f ? 1e-30f : p.scale2);
  }
  // Clear the dQ accumulator (grid-stride over float4s).
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < zero_n4; k += stride)
    reinterpret_cast<f32x4*>(p.dQacc)[k] = f32x4{0.f, 0.f, 0.f, 0.f};
}

int launch_bwd_pre(const BwdParams& p, int bf16, int d, int v, bool clear_dq, void* stream) {
  const int64_t rows = (int64_t)p.B * p.H * p.n_pad;
  const int64_t blocks = (rows + 15) / 16;
  const int64_t zero_n4 = clear_dq ? (int64_t)p.B * p.H * p.n * d / 4 : 0;
  hipStream_t st = (hipStream_t)stream;
  dim3 g((unsigned)blocks), b(256);
#define ETA_PRE(BF, DVV) hipLaunchKernelGGL((bwd_pre_kernel<BF, DVV>), g, b, 0, st, p, zero_n4)
  if (bf16) {
    if (v == 64) ETA_PRE(true, 64); else if (v == 80) ETA_PRE(true, 80); else ETA_PRE(true, 128);
  } else {
    if (v == 64) ETA_PRE(false, 64); else if (v == 80) ETA_PRE(false, 80); else ETA_PRE(false, 128);
  }
#undef ETA_PRE
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------

template <bool BF16>
__global__ __launch_bounds__(256) void bwd_post_kernel(BwdParams p, int d) {
  const int64_t q4 = d / 4;  // float4 groups per row
  const int64_t total = (int64_t)p.B * p.H * p.n * q4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total; k += stride) {
    const int64_t row = k / q4, c4 = k % q4;
    const int64_t unit = row / p.n, i = row % p.n;
    const int64_t b = unit / p.H, h = unit % p.H;
    const f32x4 x = reinterpret_cast<const f32x4*>(p.dQacc)[k];
    const int64_t off = b * p.sq[0] + h * p.sq[1] + i * p.sq[2] + 4 * c4;
    if constexpr (BF16) {
      u32x2 pk{pack_bf16x2(x[0] * p.scale, x[1] * p.scale), pack_bf16x2(x[2] * p.scale, x[3] * p.scale)};
      *reinterpret_cast<u32x2*>((char*)p.dQ + off * 2) = pk;
    } else {
      *reinterpret_cast<f32x4*>((char*)p.dQ + off * 4) =
          f32x4{x[0] * p.scale, x[1] * p.scale, x[2] * p.scale, x[3] * p.scale};
    }
  }
}

int launch_bwd_post(const BwdParams& p, int bf16, int d, void* stream) {
  const int64_t total = (int64_t)p.B * p.H * p.n * (d / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipStream_t st = (hipStream_t)stream;
  if (bf16)
    hipLaunchKernelGGL((bwd_post_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, st, p, d);
  else
    hipLaunchKernelGGL((bwd_post_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, st, p, d);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------

// Dropout keep decisions of rows [i0, i0 + rows) x keys [j0, j0 + cols) of
// one unit, one byte each: the same keep4_row draws the forward and dQ
// kernels use (the key-tile-outer kernel draws the same blocks by column).
__global__ __launch_bounds__(256) void dropout_mask_kernel(DropParams d, uint32_t unit, int64_t i0, int64_t j0,
                                                           int rows, int cols, uint8_t* out) {
  const int64_t groups = (int64_t)rows * ((cols + 3) / 4);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < groups; t += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(t / ((cols + 3) / 4)), c4 = (int)(t % ((cols + 3) / 4));
    const uint32_t bits = keep4_row(d.seed_lo, d.seed_hi, d.p8, unit, (uint32_t)(i0 + r), (uint32_t)(j0 + 4 * c4));
    for (int e = 0; e < 4 && 4 * c4 + e < cols; ++e) out[(int64_t)r * cols + 4 * c4 + e] = (bits >> e) & 1u;
  }
}

int launch_dropout_mask(const DropParams& d, uint32_t unit, int64_t i0, int64_t j0, int rows, int cols,
                        uint8_t* out, void* stream) {
  const int64_t groups = (int64_t)rows * ((cols + 3) / 4);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) return 0;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, d, unit, i0,
                     j0, rows, cols, out);
  return (int)hipGetLastError();
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }
int hip_last_launch_error() { return (int)hipGetLastError(); }

}  // namespace eta

// ---------------------------------------------------------------------------
// Opt-in launch timing: HIP events recorded on the launch stream around each
// kernel, read back (and recycled) by attn_timing_read.
// ---------------------------------------------------------------------------

#include <vector>

namespace eta {
namespace {
struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};
bool g_timing = false;
std::vector<TimedLaunch> g_pending;
std::vector<hipEvent_t> g_free;
hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void timing_begin(int kind, void* stream) {
  if (!g_timing) return;
  TimedLaunch t{kind, take_event(), take_event()};
  if (!t.start || !t.stop || hipEventRecord(t.start, (hipStream_t)stream) != hipSuccess) {
    if (t.start) g_free.push_back(t.start);
    if (t.stop) g_free.push_back(t.stop);
    return;  // this launch goes untimed
  }
  g_pending.push_back(t);
}

void timing_end(int kind, void* stream) {
  if (!g_timing || g_pending.empty() || g_pending.back().kind != kind) return;
  if (hipEventRecord(g_pending.back().stop, (hipStream_t)stream) != hipSuccess) {
    g_free.push_back(g_pending.back().start);
    g_free.push_back(g_pending.back().stop);
    g_pending.pop_back();  // a start without a stop is not a measurement
  }
}

void timing_reset() {
  for (auto& t : g_pending) {
    (void)hipEventSynchronize(t.stop);
    g_free.push_back(t.start);
    g_free.push_back(t.stop);
  }
  g_pending.clear();
}

int timing_enable(int on) {
  timing_reset();
  g_timing = on != 0;
  return 0;
}

int timing_read(double* ms, int64_t* launches) {
  int err = 0;
  for (auto& t : g_pending) {
    float el = 0.f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&el, t.start, t.stop);
    if (e != hipSuccess) {
      err = (int)e;
    } else if (t.kind >= 0 && t.kind < ATTN_KERNEL_COUNT) {
      ms[t.kind] += el;
      launches[t.kind] += 1;
    }
    g_free.push_back(t.start);
    g_free.push_back(t.stop);
  }
  g_pending.clear();
  return err;
}

}  // namespace eta
