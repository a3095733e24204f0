// Host entry points of the C ABI declared in include/attn.h: argument
// validation (complete before anything is launched), workspace planning and
// launch sequencing.  Plain C++17; all device work goes through the
// launchers in the .hip translation units.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

thread_local std::string g_last_error;

// Executed-tile counters of attn_debug_count_tiles (device words), or null.
unsigned long long* g_tile_counters = nullptr;

attn_status fail(attn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr int64_t kMaxElems = int64_t(1) << 46;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Tiles {
  int bq, bk;
  int64_t tq, tk;
};

// Key rows (nk = 0 stands for nk = n).
int64_t nkeys(const attn_problem& p) { return p.nk == 0 ? p.n : p.nk; }

// Dropout in units of 1/256 (0 = off), and its kernel parameters.
uint32_t drop_p8(const attn_problem& p) {
  const double x = std::floor(p.dropout_p * 256.0 + 0.5);
  return x >= 255.0 ? 255u : (uint32_t)x;
}
eta::DropParams drop_params(const attn_problem& p) {
  eta::DropParams d{};
  d.seed_lo = (uint32_t)(p.dropout_seed & 0xFFFFFFFFu);
  d.seed_hi = (uint32_t)(p.dropout_seed >> 32);
  d.p8 = drop_p8(p);
  d.keep_inv = d.p8 ? (float)(256.0 / (256.0 - d.p8)) : 1.f;
  return d;
}

Tiles fwd_tiles(const attn_problem& p) {
  return Tiles{eta::kFwdBq, eta::kFwdBk, cdiv(p.n, eta::kFwdBq), cdiv(nkeys(p), eta::kFwdBk)};
}
Tiles bwd_tiles(const attn_problem& p) {
  const int bq = p.dtype == ATTN_BF16 ? eta::kBwdBq : 32;
  const int bk = eta::bwd_kv2_supported(p.dtype == ATTN_BF16, p.d, p.v, p.mask_mode, p.deterministic == 0, drop_p8(p))
                     ? eta::kBwdKv2Bk
                     : eta::kBwdBk;
  return Tiles{bq, bk, cdiv(p.n, bq), cdiv(nkeys(p), bk)};
}

int64_t row_pad(int64_t n) { return cdiv(n, eta::kRowPad) * eta::kRowPad; }

int64_t mask_units(const attn_problem& p) { return p.mask_sb == 0 ? p.H : p.B * p.H; }

Tiles dq_tiles(const attn_problem& p) {
  const int64_t nk = nkeys(p);
  if (eta::bwd_dq_pipe_supported(p.dtype == ATTN_BF16, p.d, p.v, p.mask_mode, nk))
    return Tiles{eta::kDqPipeBq, eta::kDqPipeBk, cdiv(p.n, eta::kDqPipeBq), cdiv(nk, eta::kDqPipeBk)};
  return Tiles{eta::kDqBq, eta::kDqBk, cdiv(p.n, eta::kDqBq), cdiv(nk, eta::kDqBk)};
}

struct Layout {
  size_t total = 0;
  size_t off_D = 0, off_L2 = 0, off_Ls = 0, off_dQ = 0, off_map = 0, off_map_dq = 0;
  size_t ls_bytes = 0;
  size_t map_bytes = 0, map_dq_bytes = 0, dq_bytes = 0;
  int splits = 1;  // forward key-range splits
  size_t off_Op = 0, off_Lp = 0, op_bytes = 0, lp_bytes = 0;
  int dq_splits = 1;  // key-range splits of the pipelined dQ kernel
  size_t off_dqp = 0, dqp_bytes = 0;
};

int fwd_split_count(const attn_problem& p) {
  const Tiles t = fwd_tiles(p);
  return eta::fwd_splits(p.dtype == ATTN_BF16, p.d, p.v, p.B * p.H, t.tq, t.tk);
}

// Pipelined dQ kernel's key-range splits (deterministic path only).
int dq_split_count(const attn_problem& p) {
  if (!p.deterministic || !eta::bwd_dq_pipe_supported(p.dtype == ATTN_BF16, p.d, p.v, p.mask_mode, nkeys(p)))
    return 1;
  const Tiles t = dq_tiles(p);
  return eta::dq_splits(p.B * p.H, t.tq, t.tk);
}

// Backward workspace: D and L log2(e) (fp32 [B,H,n_pad] each, n_pad = n
// rounded up to kRowPad), and -L log2(e) / (c log2(e)) alike for the
// two-waves-per-SIMD dK / dV kernel; the atomic path adds the fp32 dQ accumulator, the
// deterministic path the bitmask map at the dQ tiling and, when the dQ
// kernel splits the key range, its fp32 partials (splits x [B,H,n,d]).
Layout plan(const attn_problem& p, int is_bwd) {
  Layout l;
  const int64_t units = p.B * p.H;
  const bool bitmask = p.mask_mode == ATTN_MASK_BITMASK;
  if (is_bwd) {
    const Tiles t = bwd_tiles(p), tq = dq_tiles(p);
    const bool det = p.deterministic != 0;
    const size_t rows = size_t(units) * size_t(row_pad(p.n));
    l.off_D = 0;
    l.off_L2 = align_up(size_t(4) * rows);
    l.off_Ls = l.off_L2 + align_up(size_t(4) * rows);
    l.ls_bytes = eta::bwd_kv2_supported(p.dtype == ATTN_BF16, p.d, p.v, p.mask_mode, !det, drop_p8(p))
                     ? size_t(4) * rows
                     : 0;
    l.off_dQ = l.off_Ls + align_up(l.ls_bytes);
    l.dq_bytes = det ? 0 : size_t(4) * units * p.n * p.d;
    l.off_map = l.off_dQ + align_up(l.dq_bytes);
    l.map_bytes = bitmask ? size_t(mask_units(p) * t.tq * t.tk) : 0;
    l.off_map_dq = l.off_map + align_up(l.map_bytes);
    l.map_dq_bytes = (bitmask && det) ? size_t(mask_units(p) * tq.tq * tq.tk) : 0;
    l.dq_splits = dq_split_count(p);
    l.dqp_bytes = l.dq_splits > 1 ? size_t(l.dq_splits) * size_t(units) * size_t(p.n) * size_t(p.d) * 4 : 0;
    l.off_dqp = l.off_map_dq + align_up(l.map_dq_bytes);
    l.total = l.off_dqp + align_up(l.dqp_bytes);
  } else {
    const Tiles t = fwd_tiles(p);
    l.off_map = 0;
    l.map_bytes = p.mask_mode == ATTN_MASK_BITMASK ? size_t(mask_units(p) * t.tq * t.tk) : 0;
    l.splits = fwd_split_count(p);
    const size_t rows = size_t(l.splits) * size_t(units) * size_t(p.n);
    l.op_bytes = l.splits > 1 ? rows * size_t(p.v) * 4 : 0;
    l.lp_bytes = l.splits > 1 ? rows * 4 : 0;
    l.off_Op = align_up(l.map_bytes);
    l.off_Lp = l.off_Op + align_up(l.op_bytes);
    l.total = l.off_Lp + align_up(l.lp_bytes);
  }
  return l;
}

// Checks that a [B, H, n, w] view with strides (s[0], s[1], s[2], 1) has
// non-negative, 16-byte-aligned strides and never maps two elements to one
// address.
attn_status check_view(const char* name, const int64_t s[3], int64_t B, int64_t H, int64_t n,
                       int64_t w, int es) {
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return fail(ATTN_ERR_STRIDE, "%s: negative stride %lld", name, (long long)s[i]);
    if ((s[i] * es) % 16 != 0)
      return fail(ATTN_ERR_STRIDE, "%s: stride %lld elements is not a multiple of 16 bytes", name,
                  (long long)s[i]);
  }
  // The kernels address one (batch, head) slice with 32-bit byte offsets,
  // row strides included.
  if ((n - 1) * s[2] * es + w * es > int64_t(0x7FFFFFFF) || s[2] * es > int64_t(0x7FFFFFFF))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: one head spans more than 2 GiB (n * row stride)", name);
  // Tiles also address the padding rows past the last one, up to n rounded
  // up to 256 (the tallest tile), with 32-bit offsets: those must land past
  // the buffer range, not wrap around 2^32 back into it.
  if ((n + 255) / 256 * 256 * s[2] * es + w * es > int64_t(0xFFFFFFFF))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: row stride too large for the row count (rows padded to 256 span "
                "more than 4 GiB)", name);
  struct Dim {
    int64_t size, stride;
  } dims[4] = {{B, s[0]}, {H, s[1]}, {n, s[2]}, {w, 1}};
  Dim act[4];
  int k = 0;
  for (auto& d : dims)
    if (d.size > 1) act[k++] = d;
  std::sort(act, act + k, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
  int64_t span = 1;  // elements covered by the smaller dims
  for (int i = 0; i < k; ++i) {
    if (act[i].stride < span)
      return fail(ATTN_ERR_STRIDE, "%s: strides make elements overlap", name);
    span = act[i].stride * (act[i].size - 1) + span;
  }
  return ATTN_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range view_range(const void* ptr, const int64_t s[3], int64_t B, int64_t H, int64_t n, int64_t w,
                 int es) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(ptr);
  const int64_t last = (B - 1) * s[0] + (H - 1) * s[1] + (n - 1) * s[2] + (w - 1);
  return Range{base, base + uintptr_t(last + 1) * es};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

attn_status validate_problem(const attn_problem* p) {
  if (!p) return fail(ATTN_ERR_NULL, "problem pointer is NULL");
  if (p->B < 1 || p->H < 1 || p->n < 1 || p->d < 1 || p->v < 1)
    return fail(ATTN_ERR_SHAPE, "B, H, n, d, v must be >= 1 (got %lld %lld %lld %lld %lld)",
                (long long)p->B, (long long)p->H, (long long)p->n, (long long)p->d, (long long)p->v);
  if (p->nk < 0) return fail(ATTN_ERR_SHAPE, "nk must be >= 1 (or 0 for nk = n)");
  const int64_t nk = nkeys(*p);
  if (p->n > (int64_t(1) << 30) || nk > (int64_t(1) << 30) || p->B * p->H > (int64_t(1) << 24) ||
      p->B * p->H * std::max(p->n, nk) > kMaxElems / std::max(p->d, p->v))
    return fail(ATTN_ERR_SHAPE, "problem too large");
  if (p->dtype != ATTN_F32 && p->dtype != ATTN_BF16)
    return fail(ATTN_ERR_DTYPE, "unknown dtype %d", p->dtype);
  if (p->mask_mode < ATTN_MASK_NONE || p->mask_mode > ATTN_MASK_BITMASK)
    return fail(ATTN_ERR_MASK, "unknown mask mode %d", p->mask_mode);
  if (!eta::supported_dims(p->d, p->v))
    return fail(ATTN_ERR_UNSUPPORTED, "(d, v) = (%lld, %lld) not compiled; supported: (64,64) (80,80) "
                "(128,128) (64,128)", (long long)p->d, (long long)p->v);
  if (p->deterministic != 0 && p->deterministic != 1)
    return fail(ATTN_ERR_UNSUPPORTED, "deterministic must be 0 or 1");
  if (p->reserved != 0) return fail(ATTN_ERR_UNSUPPORTED, "reserved field must be 0");
  if (!std::isfinite(p->scale)) return fail(ATTN_ERR_SHAPE, "scale must be finite");
  if (p->causal_offset != 0 && p->mask_mode != ATTN_MASK_CAUSAL)
    return fail(ATTN_ERR_MASK, "causal_offset applies to the causal mask only");
  if (p->causal_offset > (int64_t(1) << 30) || p->causal_offset < -(int64_t(1) << 30))
    return fail(ATTN_ERR_SHAPE, "|causal_offset| must be <= 2^30");
  if (!(p->dropout_p >= 0.0 && p->dropout_p < 1.0))
    return fail(ATTN_ERR_SHAPE, "dropout_p must be in [0, 1)");
  if (p->mask_mode == ATTN_MASK_BITMASK) {
    if (!p->mask) return fail(ATTN_ERR_MASK, "bitmask mode needs a mask");
    if (reinterpret_cast<uintptr_t>(p->mask) % 4)
      return fail(ATTN_ERR_STRIDE, "mask pointer must be 4-byte aligned");
    const int64_t words = (nk + 31) / 32;
    if (p->mask_si < words || p->mask_sh < 0 || p->mask_sb < 0)
      return fail(ATTN_ERR_MASK, "mask strides invalid (row stride %lld < %lld words?)",
                  (long long)p->mask_si, (long long)words);
  }
  const int es = p->dtype == ATTN_BF16 ? 2 : 4;
  attn_status st;
  if ((st = check_view("Q", p->sq, p->B, p->H, p->n, p->d, es)) != ATTN_OK) return st;
  if ((st = check_view("K", p->sk, p->B, p->H, nk, p->d, es)) != ATTN_OK) return st;
  if ((st = check_view("V", p->sv, p->B, p->H, nk, p->v, es)) != ATTN_OK) return st;
  if ((st = check_view("O", p->so, p->B, p->H, p->n, p->v, es)) != ATTN_OK) return st;
  return ATTN_OK;
}

// The backward's extra limit: on the atomic path the fused kernel addresses
// one head's fp32 dQ accumulator with 32-bit offsets.
attn_status validate_bwd(const attn_problem* p) {
  attn_status st = validate_problem(p);
  if (st != ATTN_OK) return st;
  if (!p->deterministic && p->n * p->d * 4 > int64_t(0x7FFFFFFF))
    return fail(ATTN_ERR_UNSUPPORTED, "atomic dQ path: one head's fp32 dQ accumulator (n * d * 4 bytes) exceeds "
                "2 GiB; use the deterministic path");
  return ATTN_OK;
}

attn_status check_ptr(const char* name, const void* ptr) {
  if (!ptr) return fail(ATTN_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16) return fail(ATTN_ERR_STRIDE, "%s is not 16-byte aligned", name);
  return ATTN_OK;
}

attn_status check_workspace(const Layout& l, const void* ws, size_t ws_bytes) {
  if (l.total == 0) return ATTN_OK;
  if (!ws) return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", l.total);
  if (ws_bytes < l.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, l.total);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return ATTN_OK;
}

attn_status hip_status(int err, const char* what) {
  if (err == 0) return ATTN_OK;
  return fail(ATTN_ERR_HIP, "%s: %s", what, eta::hip_error_string(err));
}

void fill_common(const attn_problem& p, int64_t sq[3], int64_t sk[3], int64_t sv[3], int64_t so[3]) {
  for (int i = 0; i < 3; ++i) {
    sq[i] = p.sq[i];
    sk[i] = p.sk[i];
    sv[i] = p.sv[i];
    so[i] = p.so[i];
  }
}

eta::MapParams map_params(const attn_problem& p, const Tiles& t, uint8_t* map, int units) {
  eta::MapParams m{};
  m.mask = p.mask;
  m.mask_sb = p.mask_sb;
  m.mask_sh = p.mask_sh;
  m.mask_si = p.mask_si;
  m.map = map;
  m.n = p.n;
  m.nk = nkeys(p);
  m.coff = p.causal_offset;
  m.B = (int32_t)p.B;
  m.H = (int32_t)p.H;
  m.units = units;
  m.bq = t.bq;
  m.bk = t.bk;
  m.tq = (int32_t)t.tq;
  m.tk = (int32_t)t.tk;
  m.mask_mode = p.mask_mode;
  return m;
}

int64_t pad8(int64_t x) { return (x + 7) / 8 * 8; }

// Launch through `fn`, bracketed by the opt-in timing events of class `kind`.
template <typename F>
attn_status timed(int kind, void* stream, const char* what, F&& fn) {
  eta::timing_begin(kind, stream);
  const int err = fn();
  eta::timing_end(kind, stream);
  return hip_status(err, what);
}

}  // namespace

extern "C" {

attn_status attn_workspace_size(const attn_problem* p, int is_bwd, size_t* bytes) {
  attn_status st = is_bwd ? validate_bwd(p) : validate_problem(p);
  if (st != ATTN_OK) return st;
  if (!bytes) return fail(ATTN_ERR_NULL, "bytes pointer is NULL");
  *bytes = plan(*p, is_bwd).total;
  return ATTN_OK;
}

attn_status attn_fwd(const attn_problem* p, const void* Q, const void* K, const void* V, void* O,
                     float* L, void* ws, size_t ws_bytes, void* stream) {
  attn_status st = validate_problem(p);
  if (st != ATTN_OK) return st;
  if ((st = check_ptr("Q", Q)) || (st = check_ptr("K", K)) || (st = check_ptr("V", V)) ||
      (st = check_ptr("O", O)) || (st = check_ptr("L", L)))
    return st;
  const int es = p->dtype == ATTN_BF16 ? 2 : 4;
  const int64_t Lst[3] = {p->H * p->n, p->n, 1};
  const Range rq = view_range(Q, p->sq, p->B, p->H, p->n, p->d, es);
  const Range rk = view_range(K, p->sk, p->B, p->H, nkeys(*p), p->d, es);
  const Range rv = view_range(V, p->sv, p->B, p->H, nkeys(*p), p->v, es);
  const Range ro = view_range(O, p->so, p->B, p->H, p->n, p->v, es);
  const Range rl = view_range(L, Lst, p->B, p->H, p->n, 1, 4);
  for (const Range& in : {rq, rk, rv}) {
    if (overlap(ro, in)) return fail(ATTN_ERR_ALIAS, "O overlaps an input");
    if (overlap(rl, in)) return fail(ATTN_ERR_ALIAS, "L overlaps an input");
  }
  if (overlap(ro, rl)) return fail(ATTN_ERR_ALIAS, "O overlaps L");
  const Layout lay = plan(*p, 0);
  if ((st = check_workspace(lay, ws, ws_bytes)) != ATTN_OK) return st;
  if (lay.total) {
    const Range rw{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + lay.total};
    for (const Range& r : {rq, rk, rv, ro, rl})
      if (overlap(rw, r)) return fail(ATTN_ERR_ALIAS, "workspace overlaps a tensor");
  }

  eta::hip_last_launch_error();  // clear any stale launch error
  const Tiles t = fwd_tiles(*p);
  uint8_t* map = lay.map_bytes ? reinterpret_cast<uint8_t*>(ws) + lay.off_map : nullptr;
  if (p->mask_mode == ATTN_MASK_BITMASK) {
    const eta::MapParams mp = map_params(*p, t, map, (int)mask_units(*p));
    if ((st = timed(ATTN_KERNEL_TILE_MAP, stream, "tile map launch",
                    [&] { return eta::launch_tile_map(mp, stream); })) != ATTN_OK)
      return st;
  }
  eta::FwdParams f{};
  f.Q = Q;
  f.K = K;
  f.V = V;
  f.O = O;
  f.L = L;
  f.map = map;
  f.mask = p->mask;
  f.mask_sb = p->mask_sb;
  f.mask_sh = p->mask_sh;
  f.mask_si = p->mask_si;
  fill_common(*p, f.sq, f.sk, f.sv, f.so);
  f.n = p->n;
  f.nk = nkeys(*p);
  f.coff = p->causal_offset;
  f.B = (int32_t)p->B;
  f.H = (int32_t)p->H;
  f.tq = (int32_t)t.tq;
  f.tk = (int32_t)t.tk;
  f.splits = lay.splits;
  f.Opart = lay.op_bytes ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + lay.off_Op) : nullptr;
  f.Lpart = lay.lp_bytes ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + lay.off_Lp) : nullptr;
  f.total = p->B * p->H * t.tq * f.splits;
  f.grid_pad = pad8(f.total);
  f.scale2 = (float)(p->scale * 1.4426950408889634);
  f.drop = drop_params(*p);
  f.tile_count = g_tile_counters;
  if (f.grid_pad > 0x7FFFFFFF) return fail(ATTN_ERR_SHAPE, "grid too large");
  if ((st = timed(ATTN_KERNEL_FWD, stream, "forward launch", [&] {
         return eta::launch_fwd(f, p->dtype == ATTN_BF16, (int)p->d, (int)p->v, p->mask_mode, stream);
       })) != ATTN_OK || f.splits == 1)
    return st;
  return timed(ATTN_KERNEL_FWD_MERGE, stream, "forward merge launch",
               [&] { return eta::launch_fwd_merge(f, p->dtype == ATTN_BF16, (int)p->v, stream); });
}

attn_status attn_bwd(const attn_problem* p, const void* Q, const void* K, const void* V, const void* O,
                     const void* dO, const float* L, void* dQ, void* dK, void* dV, void* ws,
                     size_t ws_bytes, void* stream) {
  attn_status st = validate_bwd(p);
  if (st != ATTN_OK) return st;
  if ((st = check_ptr("Q", Q)) || (st = check_ptr("K", K)) || (st = check_ptr("V", V)) ||
      (st = check_ptr("O", O)) || (st = check_ptr("dO", dO)) || (st = check_ptr("L", L)) ||
      (st = check_ptr("dQ", dQ)) || (st = check_ptr("dK", dK)) || (st = check_ptr("dV", dV)))
    return st;
  const int es = p->dtype == ATTN_BF16 ? 2 : 4;
  const int64_t Lst[3] = {p->H * p->n, p->n, 1};
  const Range ins[6] = {view_range(Q, p->sq, p->B, p->H, p->n, p->d, es),
                        view_range(K, p->sk, p->B, p->H, nkeys(*p), p->d, es),
                        view_range(V, p->sv, p->B, p->H, nkeys(*p), p->v, es),
                        view_range(O, p->so, p->B, p->H, p->n, p->v, es),
                        view_range(dO, p->so, p->B, p->H, p->n, p->v, es),
                        view_range(L, Lst, p->B, p->H, p->n, 1, 4)};
  const Range outs[3] = {view_range(dQ, p->sq, p->B, p->H, p->n, p->d, es),
                         view_range(dK, p->sk, p->B, p->H, nkeys(*p), p->d, es),
                         view_range(dV, p->sv, p->B, p->H, nkeys(*p), p->v, es)};
  const char* onames[3] = {"dQ", "dK", "dV"};
  for (int i = 0; i < 3; ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return fail(ATTN_ERR_ALIAS, "%s overlaps an input", onames[i]);
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return fail(ATTN_ERR_ALIAS, "%s overlaps %s", onames[i], onames[j]);
  }
  const Layout lay = plan(*p, 1);
  if ((st = check_workspace(lay, ws, ws_bytes)) != ATTN_OK) return st;
  const Range rw{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + lay.total};
  for (const Range& r : ins)
    if (overlap(rw, r)) return fail(ATTN_ERR_ALIAS, "workspace overlaps a tensor");
  for (const Range& r : outs)
    if (overlap(rw, r)) return fail(ATTN_ERR_ALIAS, "workspace overlaps a tensor");

  eta::hip_last_launch_error();
  const Tiles t = bwd_tiles(*p);
  char* wsb = reinterpret_cast<char*>(ws);
  eta::BwdParams b{};
  b.Q = Q;
  b.K = K;
  b.V = V;
  b.O = O;
  b.dO = dO;
  b.L = L;
  b.Dn = reinterpret_cast<float*>(wsb + lay.off_D);
  b.L2 = reinterpret_cast<float*>(wsb + lay.off_L2);
  b.Ls = lay.ls_bytes ? reinterpret_cast<float*>(wsb + lay.off_Ls) : nullptr;
  b.n_pad = row_pad(p->n);
  b.dQacc = lay.dq_bytes ? reinterpret_cast<float*>(wsb + lay.off_dQ) : nullptr;
  b.dQ = dQ;
  b.dK = dK;
  b.dV = dV;
  b.map = lay.map_bytes ? reinterpret_cast<uint8_t*>(wsb + lay.off_map) : nullptr;
  b.mask = p->mask;
  b.mask_sb = p->mask_sb;
  b.mask_sh = p->mask_sh;
  b.mask_si = p->mask_si;
  fill_common(*p, b.sq, b.sk, b.sv, b.so);
  b.n = p->n;
  b.nk = nkeys(*p);
  b.coff = p->causal_offset;
  b.B = (int32_t)p->B;
  b.H = (int32_t)p->H;
  b.tq = (int32_t)t.tq;
  b.tk = (int32_t)t.tk;
  b.total = p->B * p->H * t.tk;
  b.grid_pad = pad8(b.total);
  b.scale = (float)p->scale;
  b.scale2 = (float)(p->scale * 1.4426950408889634);
  b.drop = drop_params(*p);
  const bool det = p->deterministic != 0;
  const Tiles tdq = dq_tiles(*p);
  b.map_dq = lay.map_dq_bytes ? reinterpret_cast<uint8_t*>(wsb + lay.off_map_dq) : nullptr;
  b.tq_dq = (int32_t)tdq.tq;
  b.dq_splits = lay.dq_splits;
  b.dQpart = lay.dqp_bytes ? reinterpret_cast<float*>(wsb + lay.off_dqp) : nullptr;
  b.total_dq = p->B * p->H * tdq.tq * lay.dq_splits;
  b.grid_pad_dq = pad8(b.total_dq);
  b.tile_count_kv = g_tile_counters ? g_tile_counters + 1 : nullptr;
  b.tile_count_dq = g_tile_counters ? g_tile_counters + 2 : nullptr;
  if (b.grid_pad > 0x7FFFFFFF || b.grid_pad_dq > 0x7FFFFFFF) return fail(ATTN_ERR_SHAPE, "grid too large");
  const int bf = p->dtype == ATTN_BF16;
  if ((st = timed(ATTN_KERNEL_BWD_PRE, stream, "D preprocess launch",
                  [&] { return eta::launch_bwd_pre(b, bf, (int)p->d, (int)p->v, !det, stream); })) != ATTN_OK)
    return st;
  if (p->mask_mode == ATTN_MASK_BITMASK) {
    const eta::MapParams mp = map_params(*p, t, const_cast<uint8_t*>(b.map), (int)mask_units(*p));
    if ((st = timed(ATTN_KERNEL_TILE_MAP, stream, "tile map launch",
                    [&] { return eta::launch_tile_map(mp, stream); })) != ATTN_OK)
      return st;
    if (det) {
      const eta::MapParams mq = map_params(*p, tdq, const_cast<uint8_t*>(b.map_dq), (int)mask_units(*p));
      if ((st = timed(ATTN_KERNEL_TILE_MAP, stream, "tile map launch",
                      [&] { return eta::launch_tile_map(mq, stream); })) != ATTN_OK)
        return st;
    }
  }
  if ((st = timed(ATTN_KERNEL_BWD, stream, "backward launch", [&] {
         return eta::launch_bwd(b, bf, (int)p->d, (int)p->v, p->mask_mode, !det, stream);
       })) != ATTN_OK)
    return st;
  if (det) {
    if ((st = timed(ATTN_KERNEL_BWD_DQ, stream, "dQ launch", [&] {
           return eta::launch_bwd_dq(b, bf, (int)p->d, (int)p->v, p->mask_mode, stream);
         })) != ATTN_OK || b.dq_splits == 1)
      return st;
    return timed(ATTN_KERNEL_BWD_DQ_MERGE, stream, "dQ merge launch",
                 [&] { return eta::launch_bwd_dq_merge(b, (int)p->d, stream); });
  }
  return timed(ATTN_KERNEL_BWD_POST, stream, "dQ conversion launch",
               [&] { return eta::launch_bwd_post(b, bf, (int)p->d, stream); });
}

attn_status attn_bwd_noalloc(const attn_problem* p, const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* L, void* dQ, void* dK, void* dV, void* stream) {
  attn_status st = validate_bwd(p);
  if (st != ATTN_OK) return st;
  if ((st = check_ptr("Q", Q)) || (st = check_ptr("K", K)) || (st = check_ptr("V", V)) ||
      (st = check_ptr("O", O)) || (st = check_ptr("dO", dO)) || (st = check_ptr("L", L)) ||
      (st = check_ptr("dQ", dQ)) || (st = check_ptr("dK", dK)) || (st = check_ptr("dV", dV)))
    return st;
  const size_t need = plan(*p, 1).total, cap = eta::scratch_capacity();
  if (need > cap)
    return fail(ATTN_ERR_WORKSPACE,
                "attn_bwd_noalloc: this problem needs %zu bytes of scratch, more than the %zu-byte static "
                "buffer; call attn_bwd with a workspace of attn_workspace_size bytes",
                need, cap);
  void* ws = nullptr;
  if ((st = hip_status(eta::scratch_address(&ws), "static scratch address")) != ATTN_OK) return st;
  return attn_bwd(p, Q, K, V, O, dO, L, dQ, dK, dV, ws, cap, stream);
}

attn_status attn_debug_tile_map(const attn_problem* p, int is_bwd, uint8_t* map_dev, size_t map_bytes,
                                int32_t* bq, int32_t* bk, int32_t* tq, int32_t* tk, void* ws,
                                size_t ws_bytes, void* stream) {
  (void)ws;  // reserved
  (void)ws_bytes;
  attn_status st = validate_problem(p);
  if (st != ATTN_OK) return st;
  if (!bq || !bk || !tq || !tk) return fail(ATTN_ERR_NULL, "size outputs must not be NULL");
  if (is_bwd < 0 || is_bwd > 2) return fail(ATTN_ERR_SHAPE, "is_bwd must be 0, 1 or 2");
  const Tiles t = is_bwd == 2 ? dq_tiles(*p) : is_bwd ? bwd_tiles(*p) : fwd_tiles(*p);
  *bq = t.bq;
  *bk = t.bk;
  *tq = (int32_t)t.tq;
  *tk = (int32_t)t.tk;
  if (!map_dev) return ATTN_OK;
  const int units = p->mask_mode == ATTN_MASK_BITMASK ? (int)mask_units(*p) : 1;
  const size_t need = size_t(units) * t.tq * t.tk;
  if (map_bytes < need) return fail(ATTN_ERR_WORKSPACE, "map buffer too small: %zu < %zu", map_bytes, need);
  eta::hip_last_launch_error();
  const eta::MapParams mp = map_params(*p, t, map_dev, units);
  return hip_status(eta::launch_tile_map(mp, stream), "tile map launch");
}

attn_status attn_debug_dropout_mask(const attn_problem* p, int64_t b, int64_t h, int64_t i0, int64_t j0,
                                    int32_t rows, int32_t cols, uint8_t* out_dev, size_t out_bytes,
                                    void* stream) {
  attn_status st = validate_problem(p);
  if (st != ATTN_OK) return st;
  if (drop_p8(*p) == 0) return fail(ATTN_ERR_UNSUPPORTED, "dropout is not enabled in this problem");
  if (!out_dev) return fail(ATTN_ERR_NULL, "out_dev is NULL");
  if (b < 0 || b >= p->B || h < 0 || h >= p->H) return fail(ATTN_ERR_SHAPE, "unit (b, h) out of range");
  if (rows < 1 || cols < 1 || i0 < 0 || j0 < 0 || i0 % 4 || j0 % 4 || i0 + rows > (int64_t(1) << 31) ||
      j0 + cols > (int64_t(1) << 31))
    return fail(ATTN_ERR_SHAPE, "rows, cols >= 1 and i0, j0 non-negative multiples of 4 are required");
  if (out_bytes < size_t(rows) * size_t(cols))
    return fail(ATTN_ERR_WORKSPACE, "out buffer too small: %zu < %zu", out_bytes, size_t(rows) * size_t(cols));
  eta::hip_last_launch_error();
  return hip_status(eta::launch_dropout_mask(drop_params(*p), (uint32_t)(b * p->H + h), i0, j0, rows, cols,
                                             out_dev, stream),
                    "dropout mask launch");
}

attn_status attn_debug_count_tiles(uint64_t* counters_dev) {
  if (reinterpret_cast<uintptr_t>(counters_dev) % 8)
    return fail(ATTN_ERR_STRIDE, "tile counters must be 8-byte aligned");
  g_tile_counters = reinterpret_cast<unsigned long long*>(counters_dev);
  return ATTN_OK;
}

const char* attn_status_str(int s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid shape";
    case ATTN_ERR_STRIDE: return "invalid stride or alignment";
    case ATTN_ERR_DTYPE: return "invalid dtype";
    case ATTN_ERR_MASK: return "invalid mask";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "invalid workspace";
    case ATTN_ERR_ALIAS: return "output aliases another buffer";
    case ATTN_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

attn_status attn_timing_enable(int on) {
  eta::timing_enable(on);
  return ATTN_OK;
}

attn_status attn_timing_read(double* ms, int64_t* launches) {
  if (!ms || !launches) return fail(ATTN_ERR_NULL, "timing outputs must not be NULL");
  for (int i = 0; i < ATTN_KERNEL_COUNT; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  return hip_status(eta::timing_read(ms, launches), "timing read");
}

attn_status attn_timing_reset(void) {
  eta::timing_reset();
  return ATTN_OK;
}

int32_t attn_version(void) { return 600; }

}  // extern "C"
