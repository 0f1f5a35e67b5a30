// C ABI of libmao: host-side validation, workspace carving and the ordering
// of the kernels of each optimizer step on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

#include "common.hpp"
#include "elementwise.hpp"
#include "gemm.hpp"
#include "tiled.hpp"
#include "qr.hpp"
#include "eigh.hpp"
#include "observe.hpp"

namespace mao {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

namespace {

#define MAO_FAIL(code, ...)       \
  do {                            \
    ::mao::set_error(__VA_ARGS__); \
    return (code);                \
  } while (0)

size_t dtype_size(int dt) { return dt == MAO_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == MAO_F32 || dt == MAO_BF16; }
bool finite(float x) { return isfinite(x) != 0; }

// Bytes a buffer touches: the interval [lo, hi), and for a strided matrix
// view whose every row starts at the same offset modulo the row pitch (one
// matrix, or a batch stride that is a multiple of the pitch) the pitch and the
// bytes each row covers, so that column views of one wider buffer (a fused
// QKV weight split into its logical matrices) are told apart exactly.
struct Range {
  uintptr_t lo, hi;
  uint64_t pitch = 0, span = 0;  // pitch 0: no row structure known
};

Range mat_range(const void* p, int64_t count, int64_t rows, int64_t cols, int64_t ld,
                int64_t stride, size_t es) {
  const int64_t last = (count - 1) * stride + (rows - 1) * ld + cols;
  Range r{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(last * (int64_t)es)};
  if (count == 1 || stride % ld == 0) {
    r.pitch = (uint64_t)(ld * (int64_t)es);
    r.span = (uint64_t)(cols * (int64_t)es);
  }
  return r;
}

bool overlap(Range a, Range b) {
  if (!(a.lo < b.hi && b.lo < a.hi)) return false;
  if (a.pitch == 0 || a.pitch != b.pitch) return true;
  // rows of a cover [a.lo mod pitch, + a.span) on the circle of one pitch,
  // rows of b [b.lo mod pitch, + b.span): disjoint arcs never share a byte
  const uint64_t P = a.pitch;
  const uint64_t d = ((uint64_t)(b.lo % P) + P - (uint64_t)(a.lo % P)) % P;
  return !(d >= a.span && d + b.span <= P);
}

mao_status check_mat(const char* name, const void* data, int64_t rows, int64_t cols, int64_t ld,
                     int dtype, bool f32_only) {
  if (!data) MAO_FAIL(MAO_E_NULL, "%s: NULL data", name);
  if (rows < 1 || cols < 1) MAO_FAIL(MAO_E_SHAPE, "%s: rows=%lld cols=%lld", name, (long long)rows, (long long)cols);
  if (rows > (1 << 20) || cols > (1 << 20)) MAO_FAIL(MAO_E_SHAPE, "%s: dimension above 2^20", name);
  if (!dtype_ok(dtype) || (f32_only && dtype != MAO_F32)) MAO_FAIL(MAO_E_DTYPE, "%s: unsupported dtype %d", name, dtype);
  if (ld < cols || ld % 8 != 0) MAO_FAIL(MAO_E_LAYOUT, "%s: ld=%lld (cols=%lld) must be >= cols and a multiple of 8", name, (long long)ld, (long long)cols);
  if ((uintptr_t)data % 16 != 0) MAO_FAIL(MAO_E_LAYOUT, "%s: data not 16-byte aligned", name);
  return MAO_OK;
}

mao_status check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return MAO_OK;
  if (!ws) MAO_FAIL(MAO_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)ws % 256 != 0) MAO_FAIL(MAO_E_WORKSPACE, "workspace not 256-byte aligned");
  if (have < need) MAO_FAIL(MAO_E_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return MAO_OK;
}

mao_status check_beta(const char* name, float b) {
  if (!finite(b) || b < 0.f || b >= 1.f) MAO_FAIL(MAO_E_HPARAM, "%s=%g outside [0, 1)", name, (double)b);
  return MAO_OK;
}

// ---------------------------------------------------------------------------
// Muon
// ---------------------------------------------------------------------------

struct MuonGroupBufs {
  int rows, cols, a, b, count;
  bool wide;  // rows <= cols
  bool t32;   // X, A, Bm tiled (tiled.hpp) between iterations
  int64_t ap, bp;  // a, b padded to whole 256 x 256 tiles (tiled storage)
  int64_t ldx, ldxt, lda;
  void* X[2];
  void* Xt[2];
  void* A;
  void* Bm;
  float* partial;
  int nrb;
  float* scale;
  float *ss_r, *ss_c, *rs, *cs, *sq;
};

// The bf16 Newton-Schulz products keep X, A and Bm tiled (tiled.hpp) when
// they run on the 256 x 256 kernel anyway: at least one iteration and 128 or
// more 256 x 256 tiles in the product B X over all groups.
bool muon_tiled(int ng, const int64_t* rows, const int64_t* cols, const int64_t* count,
                const mao_muon_hparams* hp) {
  if (hp->ns_dtype != MAO_BF16 || hp->ns_steps < 1) return false;
  int64_t tiles = 0;
  for (int g = 0; g < ng; ++g) tiles += count[g] * ceil_div(rows[g], 256) * ceil_div(cols[g], 256);
  return tiles >= 128;
}

void carve_muon(Carver& c, int ng, const int64_t* rows, const int64_t* cols, const int64_t* count,
                const mao_muon_hparams* hp, MuonGroupBufs* out) {
  const size_t es = dtype_size(hp->ns_dtype);
  const bool t32 = muon_tiled(ng, rows, cols, count, hp);
  for (int g = 0; g < ng; ++g) {
    MuonGroupBufs& B = out[g];
    B.rows = (int)rows[g];
    B.cols = (int)cols[g];
    B.count = (int)count[g];
    B.wide = B.rows <= B.cols;
    B.a = std::min(B.rows, B.cols);
    B.b = std::max(B.rows, B.cols);
    B.ldx = ws_ld(B.b);
    B.ldxt = ws_ld(B.a);
    B.lda = ws_ld(B.a);
    B.t32 = t32;
    B.ap = t32_pad(B.a);
    B.bp = t32_pad(B.b);
    // X[k] holds the tiled iterate, and the row-major result after the last
    // iteration: room for either
    const size_t xsz = t32 ? std::max(B.a * B.ldx, B.ap * B.bp) : B.a * B.ldx;
    const size_t asz = t32 ? B.ap * B.ap : B.a * B.lda;
    for (int k = 0; k < 2; ++k) {
      B.X[k] = c.take<char>((size_t)B.count * xsz * es);
      B.Xt[k] = c.take<char>((size_t)B.count * B.b * B.ldxt * es);
    }
    B.A = c.take<char>((size_t)B.count * asz * es);
    B.Bm = c.take<char>((size_t)B.count * asz * es);
    B.nrb = rowblocks_for(B.rows, B.count);
    B.partial = c.take<float>((size_t)B.count * B.nrb);
    B.scale = c.take<float>(B.count);
    if (hp->norm_mode != MAO_NORM_NONE) {
      B.ss_r = c.take<float>((size_t)B.count * B.rows);
      B.ss_c = c.take<float>((size_t)B.count * B.cols);
      B.rs = c.take<float>((size_t)B.count * B.rows);
      B.cs = c.take<float>((size_t)B.count * B.cols);
      B.sq = c.take<float>((size_t)B.count * std::max(B.rows, B.cols));
    } else {
      B.ss_r = B.ss_c = B.rs = B.cs = B.sq = nullptr;
    }
  }
}

mao_status check_muon_hp(const mao_muon_hparams* hp) {
  if (!hp) MAO_FAIL(MAO_E_NULL, "hparams is NULL");
  if (!finite(hp->lr) || hp->lr < 0.f) MAO_FAIL(MAO_E_HPARAM, "lr=%g", (double)hp->lr);
  MAO_TRY(check_beta("mu", hp->mu));
  if (!finite(hp->weight_decay) || hp->weight_decay < 0.f) MAO_FAIL(MAO_E_HPARAM, "weight_decay=%g", (double)hp->weight_decay);
  if (!finite(hp->eps) || hp->eps <= 0.f) MAO_FAIL(MAO_E_HPARAM, "eps=%g must be > 0", (double)hp->eps);
  if (hp->ns_steps < 0 || hp->ns_steps > 64) MAO_FAIL(MAO_E_HPARAM, "ns_steps=%d outside 0..64", hp->ns_steps);
  if (hp->ns_dtype != MAO_F32 && hp->ns_dtype != MAO_BF16) MAO_FAIL(MAO_E_DTYPE, "ns_dtype=%d", hp->ns_dtype);
  if (hp->norm_mode < 0 || hp->norm_mode > 4) MAO_FAIL(MAO_E_HPARAM, "norm_mode=%d", hp->norm_mode);
  if (hp->norm_mode != 0 && (!finite(hp->norm_eps) || hp->norm_eps <= 0.f)) MAO_FAIL(MAO_E_HPARAM, "norm_eps=%g", (double)hp->norm_eps);
  if (hp->ns_coeffs) {
    for (int i = 0; i < 3 * hp->ns_steps; ++i)
      if (!finite(hp->ns_coeffs[i])) MAO_FAIL(MAO_E_HPARAM, "ns_coeffs[%d] not finite", i);
  }
  return MAO_OK;
}

mao_status check_batch(const char* name, const mao_batch& b, bool f32_only) {
  MAO_TRY(check_mat(name, b.data, b.rows, b.cols, b.ld, b.dtype, f32_only));
  if (b.count < 1) MAO_FAIL(MAO_E_SHAPE, "%s: count=%lld", name, (long long)b.count);
  if (b.count > 1 && b.stride < b.rows * b.ld) MAO_FAIL(MAO_E_LAYOUT, "%s: stride=%lld < rows*ld", name, (long long)b.stride);
  if (b.count > 1 && b.stride % 8 != 0) MAO_FAIL(MAO_E_LAYOUT, "%s: stride must be a multiple of 8", name);
  return MAO_OK;
}

Range batch_range(const mao_batch& b) {
  return mat_range(b.data, b.count, b.rows, b.cols, b.ld, b.count > 1 ? b.stride : 0, dtype_size(b.dtype));
}

mao_status validate_muon(int32_t ng, const mao_batch* W, const mao_batch* G, const mao_batch* M,
                         const mao_muon_hparams* hp, const mao_batch* out) {
  MAO_TRY(check_muon_hp(hp));
  if (ng < 1 || ng > MAO_MAX_GROUPS) MAO_FAIL(MAO_E_SHAPE, "ngroups=%d outside 1..%d", ng, MAO_MAX_GROUPS);
  if (!W || !G || !M) MAO_FAIL(MAO_E_NULL, "W, G or M array is NULL");
  std::vector<Range> ranges;
  for (int g = 0; g < ng; ++g) {
    MAO_TRY(check_batch("W", W[g], false));
    MAO_TRY(check_batch("G", G[g], false));
    MAO_TRY(check_batch("M", M[g], true));
    if (G[g].rows != W[g].rows || G[g].cols != W[g].cols || M[g].rows != W[g].rows ||
        M[g].cols != W[g].cols || G[g].count != W[g].count || M[g].count != W[g].count)
      MAO_FAIL(MAO_E_SHAPE, "group %d: W, G, M shapes or counts differ", g);
    ranges.push_back(batch_range(W[g]));
    ranges.push_back(batch_range(G[g]));
    ranges.push_back(batch_range(M[g]));
    if (out && out[g].data) {
      MAO_TRY(check_batch("update_out", out[g], true));
      if (out[g].rows != W[g].rows || out[g].cols != W[g].cols || out[g].count != W[g].count)
        MAO_FAIL(MAO_E_SHAPE, "group %d: update_out shape differs from W", g);
      ranges.push_back(batch_range(out[g]));
    }
  }
  for (size_t i = 0; i < ranges.size(); ++i)
    for (size_t j = i + 1; j < ranges.size(); ++j)
      if (overlap(ranges[i], ranges[j])) MAO_FAIL(MAO_E_ALIAS, "buffers %zu and %zu overlap", i, j);
  return MAO_OK;
}

size_t muon_ws(int32_t ng, const mao_batch* W, const mao_muon_hparams* hp) {
  int64_t rows[MAO_MAX_GROUPS], cols[MAO_MAX_GROUPS], count[MAO_MAX_GROUPS];
  for (int g = 0; g < ng; ++g) {
    rows[g] = W[g].rows;
    cols[g] = W[g].cols;
    count[g] = W[g].count;
  }
  MuonGroupBufs bufs[MAO_MAX_GROUPS];
  Carver c(nullptr);
  carve_muon(c, ng, rows, cols, count, hp, bufs);
  return c.used + 256;
}

// Benchmark instrumentation of a memory-bound pass: HIP events around it
// when timing is on, tagged TAG_ELEMWISE with the bytes it must move.
struct PassTimer {
  hipStream_t s;
  double bytes;
  void* ev = nullptr;
  PassTimer(hipStream_t s_, double b, bool on = true) : s(s_), bytes(b) {
    if (on && timing_on()) timing_record_begin(s, &ev);
  }
  ~PassTimer() {
    if (ev) timing_record_end(s, ev, TAG_ELEMWISE, bytes);
  }
};

mao_status run_muon(int32_t ng, const mao_batch* W, const mao_batch* G, const mao_batch* M,
                    const mao_muon_hparams* hp, void* ws, const mao_batch* out, hipStream_t s) {
  int64_t rows[MAO_MAX_GROUPS], cols[MAO_MAX_GROUPS], count[MAO_MAX_GROUPS];
  for (int g = 0; g < ng; ++g) {
    rows[g] = W[g].rows;
    cols[g] = W[g].cols;
    count[g] = W[g].count;
  }
  MuonGroupBufs bufs[MAO_MAX_GROUPS];
  Carver c(ws);
  carve_muon(c, ng, rows, cols, count, hp, bufs);
  const int xdt = hp->ns_dtype;
  const int xflags = xdt == MAO_F32 ? (GF_D_F32 | GF_C0_F32) : 0;
  // bf16: the product B X reads X as its K x N operand, so only X (wide
  // orientation) is kept between iterations; fp32 keeps X and X^T (both
  // operands K-contiguous). The final update needs X^T too when W is tall or
  // Muon+ sums along the other axis: then the last iteration also writes it.
  const bool kmajor = xdt == MAO_BF16;
  auto need_t = [&](const MuonGroupBufs& B) { return !kmajor || !B.wide || hp->norm_mode != MAO_NORM_NONE; };

  // momentum, norm, X0 (and X0^T where it is read)
  for (int g = 0; g < ng; ++g) {
    MuonGroupBufs& B = bufs[g];
    const int64_t mstride = M[g].count > 1 ? M[g].stride : 0;
    const int64_t gstride = G[g].count > 1 ? G[g].stride : 0;
    const double elems = (double)B.rows * B.cols * B.count;
    {
      // M read and written (fp32), G read
      PassTimer pt(s, elems * (8.0 + dtype_size(G[g].dtype)));
      MAO_TRY(ema_sumsq(view(M[g].data, M[g].ld, mstride), view(G[g].data, G[g].ld, gstride),
                        G[g].dtype, B.rows, B.cols, B.count, hp->mu, B.partial, B.nrb, s));
      MAO_TRY(finalize_inv_norm(B.partial, B.nrb, B.count, hp->eps, B.scale, s));
    }
    if (B.t32) {
      PassTimer pt(s, elems * (4.0 + 2.0));  // M read, X0 written (bf16)
      MAO_TRY(scale_cast_tiled(view(M[g].data, M[g].ld, mstride), B.rows, B.cols, B.count, B.scale,
                               !B.wide, B.X[0], B.ap, B.bp, B.ap * B.bp, s));
      continue;
    }
    View xa = view(B.X[0], B.ldx, (int64_t)B.a * B.ldx);
    View xb = (!kmajor || (hp->ns_steps == 0 && need_t(B))) ? view(B.Xt[0], B.ldxt, (int64_t)B.b * B.ldxt)
                                                             : view(nullptr, 0, 0);
    // M read, X0 (and X0^T where it is read) written
    PassTimer pt(s, elems * (4.0 + (xb.p ? 2.0 : 1.0) * dtype_size(xdt)));
    MAO_TRY(scale_cast_transpose(view(M[g].data, M[g].ld, mstride), B.rows, B.cols, B.count,
                                 B.scale, B.wide ? xa : xb, B.wide ? xb : xa, xdt, s));
  }

  // Newton-Schulz: A = X X^T; Bm = b A + c A A; X' = a X + Bm X
  for (int k = 0; k < hp->ns_steps; ++k) {
    const float ca = hp->ns_coeffs ? hp->ns_coeffs[3 * k + 0] : 15.f / 8.f;
    const float cb = hp->ns_coeffs ? hp->ns_coeffs[3 * k + 1] : -10.f / 8.f;
    const float cc = hp->ns_coeffs ? hp->ns_coeffs[3 * k + 2] : 3.f / 8.f;
    const int cur = k & 1, nxt = cur ^ 1;
    GemmProblem p[MAO_MAX_GROUPS];
    const bool last = k + 1 == hp->ns_steps;
    if (bufs[0].t32) {
      // tiled: a I joins the square step, Bm = a I + b A + c A A, so the
      // product X' = Bm X reads no C0; the last one writes X row-major (and
      // X^T where it is read)
      for (int g = 0; g < ng; ++g) {
        MuonGroupBufs& B = bufs[g];
        const int64_t sx = B.ap * B.bp, sa = B.ap * B.ap;
        p[g] = gemm_problem(B.a, B.a, B.b, 1.f, B.X[cur], B.bp, B.X[cur], B.bp, 0.f, nullptr, 0,
                            B.A, B.ap, GF_SYRK | GF_T32 | GF_D_T32);
        p[g].batch = B.count;
        p[g].sA = p[g].sB = sx;
        p[g].sD = sa;
      }
      MAO_TRY(launch_gemm(xdt, p, ng, s, TAG_NS_GRAM));
      for (int g = 0; g < ng; ++g) {
        MuonGroupBufs& B = bufs[g];
        const int64_t sa = B.ap * B.ap;
        p[g] = gemm_problem(B.a, B.a, B.a, cc, B.A, B.ap, B.A, B.ap, cb, B.A, B.ap, B.Bm, B.ap,
                            GF_SYRK | GF_T32 | GF_D_T32 | GF_C0_T32);
        p[g].dadd = ca;
        p[g].batch = B.count;
        p[g].sA = p[g].sB = p[g].sC0 = p[g].sD = sa;
      }
      MAO_TRY(launch_gemm(xdt, p, ng, s, TAG_NS_SQUARE));
      for (int g = 0; g < ng; ++g) {
        MuonGroupBufs& B = bufs[g];
        const int64_t sx = B.ap * B.bp;
        p[g] = gemm_problem(B.a, B.b, B.a, 1.f, B.Bm, B.ap, B.X[cur], B.bp, 0.f, nullptr, 0,
                            B.X[nxt], last ? B.ldx : B.bp,
                            GF_T32 | GF_B_KMAJOR | (last ? 0 : GF_D_T32));
        if (last && need_t(B)) {
          p[g].Dt = B.Xt[nxt];
          p[g].lddt = B.ldxt;
          p[g].sDt = (int64_t)B.b * B.ldxt;
        }
        p[g].batch = B.count;
        p[g].sA = B.ap * B.ap;
        p[g].sB = sx;
        p[g].sD = last ? (int64_t)B.a * B.ldx : sx;
      }
      MAO_TRY(launch_gemm(xdt, p, ng, s, TAG_NS_APPLY));
      continue;
    }
    for (int g = 0; g < ng; ++g) {
      MuonGroupBufs& B = bufs[g];
      p[g] = gemm_problem(B.a, B.a, B.b, 1.f, B.X[cur], B.ldx, B.X[cur], B.ldx, 0.f, nullptr, 0,
                          B.A, B.lda, GF_SYRK | xflags);
      p[g].batch = B.count;
      p[g].sA = p[g].sB = (int64_t)B.a * B.ldx;
      p[g].sD = (int64_t)B.a * B.lda;
    }
    MAO_TRY(launch_gemm(xdt, p, ng, s, TAG_NS_GRAM));
    for (int g = 0; g < ng; ++g) {
      MuonGroupBufs& B = bufs[g];
      p[g] = gemm_problem(B.a, B.a, B.a, cc, B.A, B.lda, B.A, B.lda, cb, B.A, B.lda, B.Bm, B.lda,
                          GF_SYRK | xflags);
      p[g].batch = B.count;
      p[g].sA = p[g].sB = p[g].sC0 = p[g].sD = (int64_t)B.a * B.lda;
    }
    MAO_TRY(launch_gemm(xdt, p, ng, s, TAG_NS_SQUARE));
    for (int g = 0; g < ng; ++g) {
      MuonGroupBufs& B = bufs[g];
      if (kmajor)
        p[g] = gemm_problem(B.a, B.b, B.a, 1.f, B.Bm, B.lda, B.X[cur], B.ldx, ca, B.X[cur], B.ldx,
                            B.X[nxt], B.ldx, xflags | GF_B_KMAJOR);
      else
        p[g] = gemm_problem(B.a, B.b, B.a, 1.f, B.Bm, B.lda, B.Xt[cur], B.ldxt, ca, B.X[cur], B.ldx,
                            B.X[nxt], B.ldx, xflags);
      if (!kmajor || (last && need_t(B))) {
        p[g].Dt = B.Xt[nxt];
        p[g].lddt = B.ldxt;
        p[g].sDt = (int64_t)B.b * B.ldxt;
      }
      p[g].batch = B.count;
      p[g].sA = (int64_t)B.a * B.lda;
      p[g].sB = kmajor ? (int64_t)B.a * B.ldx : (int64_t)B.b * B.ldxt;
      p[g].sC0 = p[g].sD = (int64_t)B.a * B.ldx;
    }
    MAO_TRY(launch_gemm(xdt, p, ng, s, TAG_NS_APPLY));
  }

  // Muon+ normalisation and the update, in W's orientation
  const int fin = hp->ns_steps & 1;
  for (int g = 0; g < ng; ++g) {
    MuonGroupBufs& B = bufs[g];
    View xa = view(B.X[fin], B.ldx, (int64_t)B.a * B.ldx);
    View xb = view(B.Xt[fin], B.ldxt, (int64_t)B.b * B.ldxt);
    View O = B.wide ? xa : xb;   // rows x cols
    View Ot = B.wide ? xb : xa;  // cols x rows
    const float* rs = nullptr;
    const float* cs = nullptr;
    const int mode = hp->norm_mode;
    const double elems = (double)B.rows * B.cols * B.count;
    // the Muon+ sums of squares read the result once per axis
    const int naxes = (mode == MAO_NORM_COL_ROW || mode == MAO_NORM_ROW_COL) ? 2 : mode != MAO_NORM_NONE;
    {
      PassTimer pt_norm(s, elems * naxes * dtype_size(xdt), naxes > 0);
      if (mode == MAO_NORM_COL || mode == MAO_NORM_COL_ROW) {
        MAO_TRY(row_sumsq(Ot, xdt, B.cols, B.rows, B.count, nullptr, B.ss_c, s));
        MAO_TRY(equalise_scales(B.ss_c, B.cols, B.count, hp->norm_eps, B.cs, B.sq, s));
        cs = B.cs;
        if (mode == MAO_NORM_COL_ROW) {
          MAO_TRY(row_sumsq(O, xdt, B.rows, B.cols, B.count, B.sq, B.ss_r, s));
          MAO_TRY(equalise_scales(B.ss_r, B.rows, B.count, hp->norm_eps, B.rs, nullptr, s));
          rs = B.rs;
        }
      } else if (mode == MAO_NORM_ROW || mode == MAO_NORM_ROW_COL) {
        MAO_TRY(row_sumsq(O, xdt, B.rows, B.cols, B.count, nullptr, B.ss_r, s));
        MAO_TRY(equalise_scales(B.ss_r, B.rows, B.count, hp->norm_eps, B.rs, B.sq, s));
        rs = B.rs;
        if (mode == MAO_NORM_ROW_COL) {
          MAO_TRY(row_sumsq(Ot, xdt, B.cols, B.rows, B.count, B.sq, B.ss_c, s));
          MAO_TRY(equalise_scales(B.ss_c, B.cols, B.count, hp->norm_eps, B.cs, nullptr, s));
          cs = B.cs;
        }
      }
    }
    const float scale = sqrtf((float)B.rows / (float)B.cols);
    View outv = view(nullptr, 0, 0);
    if (out && out[g].data) outv = view(out[g].data, out[g].ld, out[g].count > 1 ? out[g].stride : 0);
    // W read and written, the result read, the optional fp32 update written
    PassTimer pt(s, elems * (2.0 * dtype_size(W[g].dtype) + dtype_size(xdt) + (outv.p ? 4.0 : 0.0)));
    MAO_TRY(apply_update(view(W[g].data, W[g].ld, W[g].count > 1 ? W[g].stride : 0), W[g].dtype,
                         O, xdt, B.rows, B.cols, B.count, hp->lr, hp->weight_decay, scale, rs, cs,
                         outv, s));
  }
  return MAO_OK;
}

mao_batch as_batch(const mao_mat& m) {
  mao_batch b;
  b.data = m.data;
  b.count = 1;
  b.rows = m.rows;
  b.cols = m.cols;
  b.ld = m.ld;
  b.stride = m.rows * m.ld;
  b.dtype = m.dtype;
  return b;
}

// ---------------------------------------------------------------------------
// SOAP / FOAM shared helpers
// ---------------------------------------------------------------------------

struct RotBufs {
  float* Gf;   // m x n fp32 copy of G (when G is bf16)
  float* Gtf;  // n x m fp32 transpose of G
  float* EL;   // m x m  (SOAP only)
  float* ER;   // n x n
  float* S;    // max^2 QR input
  float* T2t;  // n x m
  float* Gtil; // m x n
  float* Mtil; // m x n
  float* U;    // m x n
  float* D;    // n x n (FOAM check)
  float* small;// FOAM: tau, flag, moment work
  int* flag;
  QrWork qr;
  char* eigh = nullptr;  // eigendecomposition workspace (FOAM's eigh refresh)
  // bf16 back rotation: N, the bases and SOAP's intermediate (N Q_R^T)^T
  bf16_t* Nb = nullptr;
  bf16_t* QRb = nullptr;
  bf16_t* QLb = nullptr;
  bf16_t* T2b = nullptr;
  // bf16x3 forward rotations: split operands (split3_bf16 layouts)
  bf16_t* X3 = nullptr;   // m x 3n': G (or [G | G]) and M (SOAP: M too)
  bf16_t* Y3 = nullptr;   // m x 3n': FOAM's M (its G and M products share a phase)
  bf16_t* ER3 = nullptr;  // n x 3n'
  bf16_t* EL3 = nullptr;  // m x 3m' (SOAP)
  bf16_t* T3 = nullptr;   // n x 3m' (SOAP)
  int64_t ld3m = 0, ld3n = 0;
  // bf16x3 refresh products (single-matrix calls): both operands' splits
  bf16_t* P3a = nullptr;
  bf16_t* P3b = nullptr;
  int64_t ld3p = 0;
  int64_t ldm, ldn;  // padded leading dims for m- and n-long rows
};

// own_qr: the bases E, the QR input S, FOAM's refresh flag and the QR
// workspace belong to this matrix; otherwise the caller points EL, ER, S and
// flag into the shared, size-grouped QR area of a many-matrix call.
// Optional buffers of a SOAP / FOAM step, from its hyperparameters.
struct CarveOpt {
  bool eigh = false;       // FOAM's eigendecomposition refresh
  bool back_bf16 = false;  // rotation back on bf16 MFMA
  bool fwd3 = false;       // forward rotations as bf16x3
  bool ref3 = false;       // refresh products as bf16x3
};

CarveOpt soap_opt(const mao_soap_hparams* hp) {
  CarveOpt o;
  o.back_bf16 = hp->back_rot_dtype == MAO_BF16;
  o.fwd3 = hp->fwd_rot == MAO_ROT_BF16X3;
  o.ref3 = hp->refresh_prod == MAO_ROT_BF16X3;
  return o;
}

CarveOpt foam_opt(const mao_foam_hparams* hp) {
  CarveOpt o;
  o.eigh = hp->refresh == MAO_REFRESH_EIGH;
  o.back_bf16 = hp->back_rot_dtype == MAO_BF16;
  o.fwd3 = hp->fwd_rot == MAO_ROT_BF16X3;
  o.ref3 = hp->refresh_prod == MAO_ROT_BF16X3;
  return o;
}

void carve_rot(Carver& c, int m, int n, bool soap, bool g_bf16, RotBufs& R, bool own_qr,
               const CarveOpt& o) {
  const bool eigh = o.eigh, back_bf16 = o.back_bf16, fwd3 = o.fwd3;
  R.ldm = ws_ld(m);
  R.ldn = ws_ld(n);
  const int big = std::max(m, n);
  const int64_t ldb = ws_ld(big);
  R.Gf = g_bf16 ? c.take<float>((size_t)m * R.ldn) : nullptr;
  R.Gtf = c.take<float>((size_t)n * R.ldm);
  R.EL = (soap && own_qr) ? c.take<float>((size_t)m * R.ldm) : nullptr;
  R.ER = own_qr ? c.take<float>((size_t)n * R.ldn) : nullptr;
  R.S = own_qr ? c.take<float>((size_t)big * ldb) : nullptr;
  R.T2t = c.take<float>((size_t)n * R.ldm);
  R.Gtil = c.take<float>((size_t)m * R.ldn);
  R.Mtil = c.take<float>((size_t)m * R.ldn);
  R.U = c.take<float>((size_t)m * R.ldn);
  R.D = soap ? nullptr : c.take<float>((size_t)n * R.ldn);
  R.small = soap ? nullptr : c.take<float>(64 + foam_moments_work_floats(m, n) + 2 * (size_t)n);
  R.flag = (soap || !own_qr) ? nullptr : c.take<int>(4);
  if (own_qr) R.qr = carve_qr_work(c, big);
  if (own_qr && eigh) R.eigh = c.take<char>(eigh_work_stride(n));
  if (own_qr && o.ref3) {
    R.ld3p = ws_ld(3 * split_width(big));
    R.P3a = c.take<bf16_t>((size_t)big * R.ld3p);
    R.P3b = c.take<bf16_t>((size_t)big * R.ld3p);
  }
  if (fwd3) {
    R.ld3m = ws_ld(3 * split_width(m));
    R.ld3n = ws_ld(3 * split_width(n));
    R.X3 = c.take<bf16_t>((size_t)m * R.ld3n);
    R.ER3 = c.take<bf16_t>((size_t)n * R.ld3n);
    if (soap) {
      R.EL3 = c.take<bf16_t>((size_t)m * R.ld3m);
      R.T3 = c.take<bf16_t>((size_t)n * R.ld3m);
    } else {
      R.Y3 = c.take<bf16_t>((size_t)m * R.ld3n);
    }
  }
  if (back_bf16) {
    R.Nb = c.take<bf16_t>((size_t)m * R.ldn);
    R.QRb = c.take<bf16_t>((size_t)n * R.ldn);
    if (soap) {
      R.QLb = c.take<bf16_t>((size_t)m * R.ldm);
      R.T2b = c.take<bf16_t>((size_t)n * R.ldm);
    }
  }
}

mao_status check_step_common(const mao_mat& W, const mao_mat& G, int64_t t) {
  MAO_TRY(check_mat("W", W.data, W.rows, W.cols, W.ld, W.dtype, false));
  MAO_TRY(check_mat("G", G.data, G.rows, G.cols, G.ld, G.dtype, false));
  if (G.rows != W.rows || G.cols != W.cols) MAO_FAIL(MAO_E_SHAPE, "G shape differs from W");
  if (t < 1) MAO_FAIL(MAO_E_HPARAM, "t=%lld must be >= 1", (long long)t);
  return MAO_OK;
}

mao_status check_state_mat(const char* name, const mao_mat& x, int64_t rows, int64_t cols) {
  MAO_TRY(check_mat(name, x.data, x.rows, x.cols, x.ld, x.dtype, true));
  if (x.rows != rows || x.cols != cols) MAO_FAIL(MAO_E_SHAPE, "%s is %lldx%lld, expected %lldx%lld", name, (long long)x.rows, (long long)x.cols, (long long)rows, (long long)cols);
  return MAO_OK;
}

Range mrange(const mao_mat& x) { return mat_range(x.data, 1, x.rows, x.cols, x.ld, 0, dtype_size(x.dtype)); }

mao_status check_no_overlap(std::vector<Range>& r) {
  for (size_t i = 0; i < r.size(); ++i)
    for (size_t j = i + 1; j < r.size(); ++j)
      if (overlap(r[i], r[j])) MAO_FAIL(MAO_E_ALIAS, "buffers %zu and %zu overlap", i, j);
  return MAO_OK;
}

mao_status check_adam_hp(float lr, float b1, float b2, float eps, float wd) {
  if (!finite(lr) || lr < 0.f) MAO_FAIL(MAO_E_HPARAM, "lr=%g", (double)lr);
  MAO_TRY(check_beta("beta1", b1));
  MAO_TRY(check_beta("beta2", b2));
  if (!finite(eps) || eps <= 0.f) MAO_FAIL(MAO_E_HPARAM, "eps=%g must be > 0", (double)eps);
  if (!finite(wd) || wd < 0.f) MAO_FAIL(MAO_E_HPARAM, "weight_decay=%g", (double)wd);
  return MAO_OK;
}

// Products of one phase of a many-matrix step (none reads another's result)
// are collected and launched together: products equal in shape, leading
// dimensions, scalars, flags and input type form one pointer-table batch
// (tables written into the step's workspace), up to kMaxProblems batches per
// launch. Without a batch a product launches at once.
struct GemmBatch {
  struct Item {
    GemmProblem p;
    int dtype;
  };
  std::vector<Item> items;
  const void** table = nullptr;  // device, `capacity` pointers
  int64_t capacity = 0;
};

mao_status gemm_add(GemmBatch* gb, const GemmProblem& p, int dtype, hipStream_t s) {
  if (gb == nullptr) {
    GemmProblem q = p;
    return launch_gemm(dtype, &q, 1, s);
  }
  gb->items.push_back({p, dtype});
  return MAO_OK;
}

bool same_batch(const GemmBatch::Item& a, const GemmBatch::Item& b) {
  const GemmProblem &x = a.p, &y = b.p;
  return a.dtype == b.dtype && x.M == y.M && x.N == y.N && x.K == y.K && x.lda == y.lda &&
         x.ldb == y.ldb && x.ldc0 == y.ldc0 && x.ldd == y.ldd && x.lddt == y.lddt &&
         x.alpha == y.alpha && x.beta == y.beta && x.dadd == y.dadd && x.flags == y.flags &&
         (x.C0 == nullptr) == (y.C0 == nullptr) && (x.D == nullptr) == (y.D == nullptr) &&
         (x.Dt == nullptr) == (y.Dt == nullptr) && x.batch == 1 && y.batch == 1 &&
         !x.row_scale && !y.row_scale && !x.pred && !y.pred && !x.ptab && !y.ptab;
}

mao_status gemm_flush(GemmBatch& gb, hipStream_t s) {
  const int n = (int)gb.items.size();
  if (n == 0) return MAO_OK;
  std::vector<std::vector<int>> groups;
  for (int i = 0; i < n; ++i) {
    bool placed = false;
    for (auto& g : groups)
      if (same_batch(gb.items[g[0]], gb.items[i])) {
        g.push_back(i);
        placed = true;
        break;
      }
    if (!placed) groups.push_back({i});
  }
  std::vector<const void*> tab;
  std::vector<GemmProblem> probs[2];  // fp32, bf16 inputs
  for (const auto& g : groups) {
    GemmProblem p = gb.items[g[0]].p;
    if (g.size() > 1) {
      p.batch = (int)g.size();
      p.ptab = gb.table + tab.size();
      for (int i : g) {
        const GemmProblem& q = gb.items[i].p;
        tab.insert(tab.end(), {q.A, q.B, q.C0, q.D, q.Dt});
      }
    }
    probs[gb.items[g[0]].dtype == MAO_BF16 ? 1 : 0].push_back(p);
  }
  if ((int64_t)tab.size() > gb.capacity) {
    set_error("gemm batch: %zu pointer-table entries exceed the workspace's %lld", tab.size(),
              (long long)gb.capacity);
    return MAO_E_WORKSPACE;
  }
  if (!tab.empty()) MAO_TRY(write_pointer_table(gb.table, tab.data(), (int)tab.size(), s));
  for (int d = 0; d < 2; ++d)
    for (size_t i = 0; i < probs[d].size(); i += kMaxProblems)
      MAO_TRY(launch_gemm(d ? MAO_BF16 : MAO_F32, probs[d].data() + i,
                          (int)std::min<size_t>(kMaxProblems, probs[d].size() - i), s));
  gb.items.clear();
  return MAO_OK;
}

// D = A B^T (fp32), optional transposed copy only.
mao_status nt32(int M, int N, int K, const float* A, int64_t lda, const float* B, int64_t ldb,
                float* D, int64_t ldd, float* Dt, int64_t lddt, hipStream_t s,
                const int* pred = nullptr, GemmBatch* gb = nullptr) {
  GemmProblem p = gemm_problem(M, N, K, 1.f, A, lda, B, ldb, 0.f, nullptr, 0, D, ldd, GF_D_F32);
  p.Dt = Dt;
  p.lddt = lddt;
  p.pred = pred;
  return gemm_add(gb, p, MAO_F32, s);
}

// D = A B^T (fp32 out; D or its transposed copy Dt) as bf16x3 on bf16 MFMA:
// A3 (M x 3K', or [A | A] over 2K' when A is exact in bf16) against B3 = [hi
// | hi | lo] (N x 3K'), both already split (split3_bf16); K' = split_width(K).
mao_status nt3(int M, int N, int K, const bf16_t* A3, int64_t lda3, bool a_dup, const bf16_t* B3,
               int64_t ldb3, float* D, int64_t ldd, float* Dt, int64_t lddt, hipStream_t s,
               GemmBatch* gb) {
  const int Kp = (int)split_width(K);
  GemmProblem p = gemm_problem(M, N, a_dup ? 2 * Kp : 3 * Kp, 1.f, A3, lda3,
                               a_dup ? B3 + Kp : B3, ldb3, 0.f, nullptr, 0, D, ldd, GF_D_F32);
  p.Dt = Dt;
  p.lddt = lddt;
  return gemm_add(gb, p, MAO_BF16, s);
}

// S = A B^T (k x k, fp32 operands and result) as bf16x3: A split into A3
// ([hi | lo | hi]) and B into B3 ([hi | hi | lo]), k x 3k' each at ld3.
mao_status nt3_split(int k, const float* A, int64_t lda, const float* B, int64_t ldb, float* S,
                     int64_t ldS, bf16_t* A3, bf16_t* B3, int64_t ld3, hipStream_t s,
                     GemmBatch* gb) {
  MAO_TRY(split3_bf16(view((void*)A, lda), MAO_F32, k, k, view(A3, ld3), kSplitA, s));
  MAO_TRY(split3_bf16(view((void*)B, ldb), MAO_F32, k, k, view(B3, ld3), kSplitB, s));
  return nt3(k, k, k, A3, ld3, false, B3, ld3, S, ldS, nullptr, 0, s, gb);
}

// F <- beta F + (1 - beta) X X^T (SYRK in place, fp32 F; X fp32 or bf16:
// bf16 products are exact in fp32, so both accumulate alike in fp32)
mao_status syrk_ema(int N, int K, const void* X, int64_t ldx, float beta, float* F, int64_t ldf,
                    hipStream_t s, int x_dtype = MAO_F32, GemmBatch* gb = nullptr) {
  GemmProblem p = gemm_problem(N, N, K, 1.f - beta, X, ldx, X, ldx, beta, F, ldf, F, ldf,
                               GF_SYRK | GF_D_F32 | GF_C0_F32);
  return gemm_add(gb, p, x_dtype, s);
}

}  // namespace
}  // namespace mao

using namespace mao;

extern "C" {

const char* mao_status_string(mao_status s) {
  switch (s) {
    case MAO_OK: return "ok";
    case MAO_E_NULL: return "null pointer";
    case MAO_E_SHAPE: return "bad shape";
    case MAO_E_DTYPE: return "unsupported dtype";
    case MAO_E_LAYOUT: return "bad layout or alignment";
    case MAO_E_ALIAS: return "overlapping buffers";
    case MAO_E_HPARAM: return "hyperparameter out of range";
    case MAO_E_WORKSPACE: return "workspace missing or too small";
    case MAO_E_HIP: return "HIP runtime error";
    case MAO_E_UNSUPPORTED: return "unsupported request";
  }
  return "unknown status";
}

const char* mao_last_error(void) { return g_err; }

int mao_abi_version(void) { return MAO_ABI_VERSION; }

size_t muon_workspace_size(int64_t rows, int64_t cols, const mao_muon_hparams* hp) {
  if (!hp || rows < 1 || cols < 1) return 0;
  mao_batch b = {nullptr, 1, rows, cols, round_up(cols, 8), rows * round_up(cols, 8), MAO_F32};
  return muon_ws(1, &b, hp);
}

size_t muon_batched_workspace_size(int32_t ngroups, const mao_batch* W, const mao_muon_hparams* hp) {
  if (!hp || !W || ngroups < 1 || ngroups > MAO_MAX_GROUPS) return 0;
  for (int g = 0; g < ngroups; ++g)
    if (W[g].rows < 1 || W[g].cols < 1 || W[g].count < 1) return 0;
  return muon_ws(ngroups, W, hp);
}

mao_status muon_step_batched(int32_t ngroups, const mao_batch* W, const mao_batch* G,
                             const mao_batch* M, const mao_muon_hparams* hp, void* workspace,
                             size_t workspace_bytes, const mao_batch* update_out, void* stream) {
  MAO_TRY(validate_muon(ngroups, W, G, M, hp, update_out));
  MAO_TRY(check_workspace(workspace, workspace_bytes, muon_ws(ngroups, W, hp)));
  return run_muon(ngroups, W, G, M, hp, workspace, update_out, (hipStream_t)stream);
}

mao_status muon_step(mao_mat W, mao_mat G, mao_mat M, const mao_muon_hparams* hp, void* workspace,
                     size_t workspace_bytes, float* update_out, void* stream) {
  mao_batch w = as_batch(W), g = as_batch(G), m = as_batch(M);
  mao_batch o = {update_out, 1, W.rows, W.cols, W.cols, W.rows * W.cols, MAO_F32};
  if (update_out && W.cols % 8 != 0) {
    // dense fp32 output rows are not 8-aligned: still valid, checked as a flat buffer
    o.ld = W.cols;
  }
  MAO_TRY(check_muon_hp(hp));
  if (update_out && (uintptr_t)update_out % 16 != 0) MAO_FAIL(MAO_E_LAYOUT, "update_out not 16-byte aligned");
  if (update_out && W.cols % 4 != 0) MAO_FAIL(MAO_E_LAYOUT, "update_out needs cols %% 4 == 0");
  // validate W/G/M, then the dense output separately (its ld is cols)
  MAO_TRY(validate_muon(1, &w, &g, &m, hp, nullptr));
  if (update_out) {
    std::vector<Range> r = {batch_range(w), batch_range(g), batch_range(m),
                            mat_range(update_out, 1, W.rows, W.cols, W.cols, 0, 4)};
    MAO_TRY(check_no_overlap(r));
  }
  MAO_TRY(check_workspace(workspace, workspace_bytes, muon_ws(1, &w, hp)));
  return run_muon(1, &w, &g, &m, hp, workspace, update_out ? &o : nullptr, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------

size_t soap_workspace_size(int64_t rows, int64_t cols, const mao_soap_hparams* hp) {
  if (!hp || rows < 1 || cols < 1) return 0;
  Carver c(nullptr);
  RotBufs R;
  carve_rot(c, (int)rows, (int)cols, true, true, R, true, soap_opt(hp));
  return c.used + 256;
}

}  // extern "C"

namespace {

// Argument checks of one SOAP matrix; its buffers go to rr.
mao_status validate_soap(const mao_mat& W, const mao_mat& G, const mao_soap_state* st, int64_t t,
                         const float* update_out, std::vector<Range>& rr) {
  if (!st) MAO_FAIL(MAO_E_NULL, "state is NULL");
  MAO_TRY(check_step_common(W, G, t));
  const int64_t m = W.rows, n = W.cols;
  MAO_TRY(check_state_mat("M", st->M, m, n));
  MAO_TRY(check_state_mat("V", st->V, m, n));
  MAO_TRY(check_state_mat("L", st->L, m, m));
  MAO_TRY(check_state_mat("R", st->R, n, n));
  MAO_TRY(check_state_mat("QL", st->QL, m, m));
  MAO_TRY(check_state_mat("QR", st->QR, n, n));
  if (update_out && ((uintptr_t)update_out % 16 != 0 || n % 4 != 0))
    MAO_FAIL(MAO_E_LAYOUT, "update_out must be 16-byte aligned with cols %% 4 == 0");
  for (const Range& r : {mrange(W), mrange(G), mrange(st->M), mrange(st->V), mrange(st->L),
                         mrange(st->R), mrange(st->QL), mrange(st->QR)})
    rr.push_back(r);
  if (update_out) rr.push_back(mat_range(update_out, 1, m, n, n, 0, 4));
  return MAO_OK;
}

mao_status check_soap_hp(const mao_soap_hparams* hp) {
  if (!hp) MAO_FAIL(MAO_E_NULL, "hparams is NULL");
  MAO_TRY(check_adam_hp(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay));
  if (hp->refresh_every < 0) MAO_FAIL(MAO_E_HPARAM, "refresh_every=%d", hp->refresh_every);
  if (!dtype_ok(hp->back_rot_dtype)) MAO_FAIL(MAO_E_DTYPE, "back_rot_dtype=%d", hp->back_rot_dtype);
  if (hp->fwd_rot != MAO_ROT_F32 && hp->fwd_rot != MAO_ROT_BF16X3)
    MAO_FAIL(MAO_E_HPARAM, "fwd_rot=%d", hp->fwd_rot);
  if (hp->refresh_prod != MAO_ROT_F32 && hp->refresh_prod != MAO_ROT_BF16X3)
    MAO_FAIL(MAO_E_HPARAM, "refresh_prod=%d", hp->refresh_prod);
  return MAO_OK;
}

bool soap_refresh(const mao_soap_hparams* hp, int64_t t) {
  return hp->refresh_every > 0 && ((t - 1) % hp->refresh_every) == 0;
}

// SOAP before the refresh: momentum, fp32 G and G^T, factor EMAs with the
// current gradient, E = Q^T of both bases.
mao_status soap_pre(const mao_mat& W, const mao_mat& G, const mao_soap_state* st, RotBufs& R,
                    const mao_soap_hparams* hp, GemmBatch* gb, hipStream_t s) {
  const int m = (int)W.rows, n = (int)W.cols;
  const float b1 = hp->beta1, b2 = hp->beta2;
  float* M = (float*)st->M.data;
  // 1. momentum
  MAO_TRY(ema_sumsq(view(M, st->M.ld), view(G.data, G.ld), G.dtype, m, n, 1, b1, nullptr,
                    rowblocks_for(m, 1), s));
  // 2. factor EMAs with the current gradient
  if (G.dtype == MAO_BF16) {
    // bf16 G: the SYRKs run on the bf16 MFMA path (exact products, fp32
    // accumulation); G^T in bf16 goes to T2t, which is free until the
    // rotations; the rotations take the fp32 copy of G
    MAO_TRY(cast_transpose_f32(view(G.data, G.ld), G.dtype, m, n, view(R.Gf, R.ldn),
                               view(nullptr, 0), s));
    MAO_TRY(transpose(view(G.data, G.ld), view(R.T2t, R.ldm), m, n, 1, MAO_BF16, s));
    MAO_TRY(syrk_ema(m, n, G.data, G.ld, b2, (float*)st->L.data, st->L.ld, s, MAO_BF16, gb));
    MAO_TRY(syrk_ema(n, m, R.T2t, R.ldm, b2, (float*)st->R.data, st->R.ld, s, MAO_BF16, gb));
  } else {
    MAO_TRY(cast_transpose_f32(view(G.data, G.ld), G.dtype, m, n, view(nullptr, 0),
                               view(R.Gtf, R.ldm), s));
    MAO_TRY(syrk_ema(m, n, G.data, G.ld, b2, (float*)st->L.data, st->L.ld, s, MAO_F32, gb));
    MAO_TRY(syrk_ema(n, m, R.Gtf, R.ldm, b2, (float*)st->R.data, st->R.ld, s, MAO_F32, gb));
  }
  // 3a. E = Q^T of both bases
  MAO_TRY(transpose(view(st->QL.data, st->QL.ld), view(R.EL, R.ldm), m, m, 1, MAO_F32, s));
  return transpose(view(st->QR.data, st->QR.ld), view(R.ER, R.ldn), n, n, 1, MAO_F32, s);
}

// SOAP after the refresh in seven stages (within a stage the matrices'
// products are independent): 0-3 the rotations G~ = E_L (G E_R^T) and
// M~ = E_L (M E_R^T) through the transposed intermediate T2t; 4 Adam in the
// eigenbasis (N written over G~) and T2t = (N Q_R^T)^T; 5 U = Q_L T2t^T;
// 6 the weight update.
constexpr int kSoapPostStages = 7;

mao_status soap_post(int stage, const mao_mat& W, const mao_mat& G, const mao_soap_state* st,
                     RotBufs& R, int64_t t, const mao_soap_hparams* hp, float* update_out,
                     GemmBatch* gb, hipStream_t s) {
  const int m = (int)W.rows, n = (int)W.cols;
  const float b1 = hp->beta1, b2 = hp->beta2;
  const float* M = (const float*)st->M.data;
  const int64_t ldM = st->M.ld;
  const float* Gf = G.dtype == MAO_F32 ? (const float*)G.data : R.Gf;
  const int64_t ldG = G.dtype == MAO_F32 ? G.ld : R.ldn;
  float* U = update_out ? update_out : R.U;
  const int64_t ldU = update_out ? n : R.ldn;
  const bool f3 = hp->fwd_rot == MAO_ROT_BF16X3;
  if (f3 && stage <= 3) {
    // fp32-accurate rotations as bf16x3 products (split operands)
    switch (stage) {
      case 0: {
        MAO_TRY(split3_bf16(view(R.ER, R.ldn), MAO_F32, n, n, view(R.ER3, R.ld3n), kSplitB, s));
        const bool dup = G.dtype == MAO_BF16;
        MAO_TRY(split3_bf16(view(G.data, G.ld), G.dtype, m, n, view(R.X3, R.ld3n),
                            dup ? kSplitDup : kSplitA, s));
        return nt3(m, n, n, R.X3, R.ld3n, dup, R.ER3, R.ld3n, nullptr, 0, R.T2t, R.ldm, s, gb);
      }
      case 1:
        MAO_TRY(split3_bf16(view(R.EL, R.ldm), MAO_F32, m, m, view(R.EL3, R.ld3m), kSplitA, s));
        MAO_TRY(split3_bf16(view(R.T2t, R.ldm), MAO_F32, n, m, view(R.T3, R.ld3m), kSplitB, s));
        return nt3(m, n, m, R.EL3, R.ld3m, false, R.T3, R.ld3m, R.Gtil, R.ldn, nullptr, 0, s, gb);
      case 2:
        MAO_TRY(split3_bf16(view((void*)M, ldM), MAO_F32, m, n, view(R.X3, R.ld3n), kSplitA, s));
        return nt3(m, n, n, R.X3, R.ld3n, false, R.ER3, R.ld3n, nullptr, 0, R.T2t, R.ldm, s, gb);
      default:
        MAO_TRY(split3_bf16(view(R.T2t, R.ldm), MAO_F32, n, m, view(R.T3, R.ld3m), kSplitB, s));
        return nt3(m, n, m, R.EL3, R.ld3m, false, R.T3, R.ld3m, R.Mtil, R.ldn, nullptr, 0, s, gb);
    }
  }
  switch (stage) {
    case 0: return nt32(m, n, n, Gf, ldG, R.ER, R.ldn, nullptr, 0, R.T2t, R.ldm, s, nullptr, gb);
    case 1: return nt32(m, n, m, R.EL, R.ldm, R.T2t, R.ldm, R.Gtil, R.ldn, nullptr, 0, s, nullptr, gb);
    case 2: return nt32(m, n, n, M, ldM, R.ER, R.ldn, nullptr, 0, R.T2t, R.ldm, s, nullptr, gb);
    case 3: return nt32(m, n, m, R.EL, R.ldm, R.T2t, R.ldm, R.Mtil, R.ldn, nullptr, 0, s, nullptr, gb);
    case 4: {
      const float bc1 = (float)(1.0 - pow((double)b1, (double)t));
      const float bc2 = (float)(1.0 - pow((double)b2, (double)t));
      if (hp->back_rot_dtype == MAO_BF16) {
        // N and Q_R in bf16, (N Q_R^T)^T stored in bf16 (bf16 MFMA, fp32 accumulation)
        MAO_TRY(soap_adam(view(R.Gtil, R.ldn), view(R.Mtil, R.ldn), view(st->V.data, st->V.ld),
                          m, n, b2, bc1, bc2, hp->eps, s, view(R.Nb, R.ldn)));
        MAO_TRY(scale_cast_transpose(view(st->QR.data, st->QR.ld), n, n, 1, nullptr,
                                     view(R.QRb, R.ldn), view(nullptr, 0), MAO_BF16, s));
        GemmProblem p = gemm_problem(m, n, n, 1.f, R.Nb, R.ldn, R.QRb, R.ldn, 0.f, nullptr, 0,
                                     nullptr, 0, 0);
        p.Dt = R.T2b;
        p.lddt = R.ldm;
        return gemm_add(gb, p, MAO_BF16, s);
      }
      MAO_TRY(soap_adam(view(R.Gtil, R.ldn), view(R.Mtil, R.ldn), view(st->V.data, st->V.ld), m,
                        n, b2, bc1, bc2, hp->eps, s));
      return nt32(m, n, n, R.Gtil, R.ldn, (const float*)st->QR.data, st->QR.ld, nullptr, 0, R.T2t,
                  R.ldm, s, nullptr, gb);
    }
    case 5:
      if (hp->back_rot_dtype == MAO_BF16) {
        MAO_TRY(scale_cast_transpose(view(st->QL.data, st->QL.ld), m, m, 1, nullptr,
                                     view(R.QLb, R.ldm), view(nullptr, 0), MAO_BF16, s));
        GemmProblem p = gemm_problem(m, n, m, 1.f, R.QLb, R.ldm, R.T2b, R.ldm, 0.f, nullptr, 0,
                                     U, ldU, GF_D_F32);
        return gemm_add(gb, p, MAO_BF16, s);
      }
      return nt32(m, n, m, (const float*)st->QL.data, st->QL.ld, R.T2t, R.ldm, U, ldU, nullptr, 0,
                  s, nullptr, gb);
    default:
      return apply_update(view(W.data, W.ld), W.dtype, view(U, ldU), MAO_F32, m, n, 1, hp->lr,
                          hp->weight_decay, 1.f, nullptr, nullptr, view(nullptr, 0), s);
  }
}

mao_status check_foam_hp(const mao_foam_hparams* hp) {
  if (!hp) MAO_FAIL(MAO_E_NULL, "hparams is NULL");
  MAO_TRY(check_adam_hp(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay));
  if (hp->pf < 1) MAO_FAIL(MAO_E_HPARAM, "pf=%d must be >= 1", hp->pf);
  if (!(hp->tol >= 0.f)) MAO_FAIL(MAO_E_HPARAM, "tol=%g must be >= 0", (double)hp->tol);
  if (hp->side != MAO_FOAM_INPUT && hp->side != MAO_FOAM_OUTPUT)
    MAO_FAIL(MAO_E_HPARAM, "side=%d must be 0 (input) or 1 (output)", hp->side);
  if (hp->refresh != MAO_REFRESH_QR && hp->refresh != MAO_REFRESH_EIGH)
    MAO_FAIL(MAO_E_HPARAM, "refresh=%d must be 0 (QR) or 1 (eigh)", hp->refresh);
  if (!dtype_ok(hp->back_rot_dtype)) MAO_FAIL(MAO_E_DTYPE, "back_rot_dtype=%d", hp->back_rot_dtype);
  if (hp->fwd_rot != MAO_ROT_F32 && hp->fwd_rot != MAO_ROT_BF16X3)
    MAO_FAIL(MAO_E_HPARAM, "fwd_rot=%d", hp->fwd_rot);
  if (hp->refresh_prod != MAO_ROT_F32 && hp->refresh_prod != MAO_ROT_BF16X3)
    MAO_FAIL(MAO_E_HPARAM, "refresh_prod=%d", hp->refresh_prod);
  if (hp->refresh_prod == MAO_ROT_BF16X3 && hp->refresh == MAO_REFRESH_EIGH)
    MAO_FAIL(MAO_E_UNSUPPORTED, "bf16x3 criterion products with the eigendecomposition refresh");
  return MAO_OK;
}

bool foam_eigh(const mao_foam_hparams* hp) { return hp->refresh == MAO_REFRESH_EIGH; }

bool foam_out(const mao_foam_hparams* hp) { return hp->side == MAO_FOAM_OUTPUT; }

mao_status validate_foam(const mao_mat& W, const mao_mat& G, const mao_foam_state* st, int64_t t,
                         const mao_foam_hparams* hp, const float* update_out,
                         std::vector<Range>& rr) {
  if (!st) MAO_FAIL(MAO_E_NULL, "state is NULL");
  MAO_TRY(check_step_common(W, G, t));
  const int64_t m = W.rows, n = W.cols, k = foam_out(hp) ? m : n;
  if (foam_eigh(hp) && k > kEighMaxN)
    MAO_FAIL(MAO_E_UNSUPPORTED, "eigendecomposition refresh of a %lld x %lld factor (at most %d)",
             (long long)k, (long long)k, kEighMaxN);
  MAO_TRY(check_state_mat("M", st->M, m, n));
  MAO_TRY(check_state_mat("R", st->R, k, k));
  MAO_TRY(check_state_mat("QR", st->QR, k, k));
  if (!st->r || !st->c || !st->aux) MAO_FAIL(MAO_E_NULL, "r, c or aux is NULL");
  if (((uintptr_t)st->r | (uintptr_t)st->c | (uintptr_t)st->aux) % 4 != 0) MAO_FAIL(MAO_E_LAYOUT, "r, c, aux misaligned");
  if (update_out && ((uintptr_t)update_out % 16 != 0 || n % 4 != 0))
    MAO_FAIL(MAO_E_LAYOUT, "update_out must be 16-byte aligned with cols %% 4 == 0");
  for (const Range& r : {mrange(W), mrange(G), mrange(st->M), mrange(st->R), mrange(st->QR),
                         Range{(uintptr_t)st->r, (uintptr_t)(st->r + m)},
                         Range{(uintptr_t)st->c, (uintptr_t)(st->c + n)},
                         Range{(uintptr_t)st->aux, (uintptr_t)(st->aux + 4)}})
    rr.push_back(r);
  if (update_out) rr.push_back(mat_range(update_out, 1, m, n, n, 0, 4));
  return MAO_OK;
}

bool foam_checks(const mao_foam_hparams* hp, int64_t t) { return (t - 1) % hp->pf == 0; }

// FOAM before the refresh: momentum, fp32 G and G^T, R EMA, E_R = QR^T.
//
// The output side is the input side of the transposed problem: its buffers
// are carved for (n, m), so that Gf holds G^T (n x m) and Gtf holds G
// (m x n), the factor is G G^T, r and c trade places and U leaves through the
// transposed store of the last product.
mao_status foam_pre(const mao_mat& W, const mao_mat& G, const mao_foam_state* st, RotBufs& R,
                    const mao_foam_hparams* hp, GemmBatch* gb, hipStream_t s) {
  const int m = (int)W.rows, n = (int)W.cols;
  const bool out = foam_out(hp);
  const int k = out ? m : n;  // factor size
  const float b1 = hp->beta1, b2 = hp->beta2;
  float* Rf = (float*)st->R.data;
  const int64_t ldR = st->R.ld;
  MAO_TRY(ema_sumsq(view(st->M.data, st->M.ld), view(G.data, G.ld), G.dtype, m, n, 1, b1, nullptr,
                    rowblocks_for(m, 1), s));
  if (!out) {
    MAO_TRY(cast_transpose_f32(view(G.data, G.ld), G.dtype, m, n,
                               view(G.dtype == MAO_F32 ? nullptr : R.Gf, R.ldn), view(R.Gtf, R.ldm), s));
    MAO_TRY(syrk_ema(n, m, R.Gtf, R.ldm, b2, Rf, ldR, s, MAO_F32, gb));   // R = b2 R + (1-b2) G^T G
  } else {
    const bool f32 = G.dtype == MAO_F32;
    MAO_TRY(cast_transpose_f32(view(G.data, G.ld), G.dtype, m, n,
                               view(f32 ? nullptr : R.Gtf, R.ldm), view(R.Gf, R.ldn), s));
    const float* Gr = f32 ? (const float*)G.data : R.Gtf;
    MAO_TRY(syrk_ema(m, n, Gr, f32 ? G.ld : R.ldm, b2, Rf, ldR, s, MAO_F32, gb));   // L = b2 L + (1-b2) G G^T
  }
  return transpose(view(st->QR.data, st->QR.ld), view(R.ER, R.ldn), k, k, 1, MAO_F32, s);
}

// FOAM's refresh criterion, stage by stage (factor size k): on a check step
// S = E_R R (the QR input; stage 0), D = S E_R = Q^T R Q (stage 1) and the
// off-diagonal test that sets the refresh flag (stage 2); on other steps
// stage 2 clears the flag.
// With A3 / B3 (k x 3k' at ld3) the two products run as bf16x3.
mao_status foam_criterion(int k, const mao_foam_state* st, RotBufs& R, int64_t t,
                          const mao_foam_hparams* hp, int stage, GemmBatch* gb, hipStream_t s,
                          bf16_t* A3 = nullptr, bf16_t* B3 = nullptr, int64_t ld3 = 0) {
  const bool check = foam_checks(hp, t);
  if (check && A3 && stage == 0)
    return nt3_split(k, R.ER, R.ldn, (const float*)st->R.data, st->R.ld, R.S, R.ldn, A3, B3, ld3,
                     s, gb);
  if (check && A3 && stage == 1)
    return nt3_split(k, R.S, R.ldn, R.ER, R.ldn, R.D, R.ldn, A3, B3, ld3, s, gb);
  if (stage == 0)
    return check ? nt32(k, k, k, R.ER, R.ldn, (const float*)st->R.data, st->R.ld, R.S, R.ldn,
                        nullptr, 0, s, nullptr, gb)
                 : MAO_OK;
  if (stage == 1)
    return check ? nt32(k, k, k, R.S, R.ldn, R.ER, R.ldn, R.D, R.ldn, nullptr, 0, s, nullptr, gb)
                 : MAO_OK;
  if (!check) return no_check(st->aux, R.flag, s);
  return offdiag_check(view(R.D, R.ldn), k, hp->tol, R.small + 64, st->aux, R.flag, s);
}

// FOAM after the refresh, in three phases: the rotations G_rot = G Q_R and
// M_rot = M Q_R; the factored moment, the preconditioning and the rotation
// back U = N Q_R^T; the weight update. The output side runs the transposed
// problem: G_rot^T = G^T Q_L, M_rot^T = M^T Q_L, and U = Q_L N leaves through
// the transposed store of the last product.
float* foam_u(RotBufs& R, const mao_foam_hparams* hp, int n, float* update_out, int64_t& ldU) {
  if (update_out) {
    ldU = n;
    return update_out;
  }
  ldU = foam_out(hp) ? R.ldm : R.ldn;
  return foam_out(hp) ? R.T2t : R.U;
}

mao_status foam_rotate(const mao_mat& W, const mao_mat& G, const mao_foam_state* st, RotBufs& R,
                       const mao_foam_hparams* hp, GemmBatch* gb, hipStream_t s) {
  const int m = (int)W.rows, n = (int)W.cols;
  if (hp->fwd_rot == MAO_ROT_BF16X3) {
    // problem pm x pn: G_rot = G E_R^T (input side), or G^T E_R^T (output
    // side, from G's fp32 transposed copy); M likewise
    const bool out = foam_out(hp);
    const int pm = out ? n : m, pn = out ? m : n;
    MAO_TRY(split3_bf16(view(R.ER, R.ldn), MAO_F32, pn, pn, view(R.ER3, R.ld3n), kSplitB, s));
    const bool dup = !out && G.dtype == MAO_BF16;
    if (out)
      MAO_TRY(split3_bf16(view(R.Gf, R.ldn), MAO_F32, pm, pn, view(R.X3, R.ld3n), kSplitA, s));
    else
      MAO_TRY(split3_bf16(view(G.data, G.ld), G.dtype, pm, pn, view(R.X3, R.ld3n),
                          dup ? kSplitDup : kSplitA, s));
    MAO_TRY(nt3(pm, pn, pn, R.X3, R.ld3n, dup, R.ER3, R.ld3n, R.Gtil, R.ldn, nullptr, 0, s, gb));
    if (out) {
      MAO_TRY(transpose(view(st->M.data, st->M.ld), view(R.U, R.ldn), m, n, 1, MAO_F32, s));
      MAO_TRY(split3_bf16(view(R.U, R.ldn), MAO_F32, pm, pn, view(R.Y3, R.ld3n), kSplitA, s));
    } else {
      MAO_TRY(split3_bf16(view(st->M.data, st->M.ld), MAO_F32, pm, pn, view(R.Y3, R.ld3n),
                          kSplitA, s));
    }
    return nt3(pm, pn, pn, R.Y3, R.ld3n, false, R.ER3, R.ld3n, R.Mtil, R.ldn, nullptr, 0, s, gb);
  }
  if (foam_out(hp)) {
    MAO_TRY(nt32(n, m, m, R.Gf, R.ldn, R.ER, R.ldn, R.Gtil, R.ldn, nullptr, 0, s, nullptr, gb));
    MAO_TRY(transpose(view(st->M.data, st->M.ld), view(R.U, R.ldn), m, n, 1, MAO_F32, s));
    return nt32(n, m, m, R.U, R.ldn, R.ER, R.ldn, R.Mtil, R.ldn, nullptr, 0, s, nullptr, gb);
  }
  const float* Gf = G.dtype == MAO_F32 ? (const float*)G.data : R.Gf;
  const int64_t ldG = G.dtype == MAO_F32 ? G.ld : R.ldn;
  MAO_TRY(nt32(m, n, n, Gf, ldG, R.ER, R.ldn, R.Gtil, R.ldn, nullptr, 0, s, nullptr, gb));
  return nt32(m, n, n, (const float*)st->M.data, st->M.ld, R.ER, R.ldn, R.Mtil, R.ldn, nullptr, 0,
              s, nullptr, gb);
}

mao_status foam_precondition_back(const mao_mat& W, const mao_foam_state* st, RotBufs& R,
                                  int64_t t, const mao_foam_hparams* hp, float* update_out,
                                  GemmBatch* gb, hipStream_t s) {
  const int m = (int)W.rows, n = (int)W.cols;
  const float b1 = hp->beta1, b2 = hp->beta2;
  float* tau = R.small;
  float* work = R.small + 64;
  const float bc1 = (float)(1.0 - pow((double)b1, (double)t));
  const float bc2 = (float)(1.0 - pow((double)b2, (double)t));
  int64_t ldU;
  float* U = foam_u(R, hp, n, update_out, ldU);
  const bool bb = hp->back_rot_dtype == MAO_BF16;
  // problem dimensions: the output side runs the transposed problem (n x m)
  const bool out = foam_out(hp);
  const int pm = out ? n : m, pn = out ? m : n;
  MAO_TRY(foam_moments(view(R.Gtil, R.ldn), pm, pn, b2, bc2, (const float*)st->R.data, st->R.ld,
                       out ? st->c : st->r, out ? st->r : st->c, work, tau, st->aux, s));
  MAO_TRY(foam_precondition(view(R.Mtil, R.ldn), pm, pn, out ? st->c : st->r,
                            out ? st->r : st->c, tau, bc1, bc2, hp->eps, s,
                            bb ? view(R.Nb, R.ldn) : view(nullptr, 0)));
  // rotation back U = N Q_R^T (output side: U^T, through the transposed store)
  GemmProblem p;
  if (bb) {
    MAO_TRY(scale_cast_transpose(view(st->QR.data, st->QR.ld), pn, pn, 1, nullptr,
                                 view(R.QRb, R.ldn), view(nullptr, 0), MAO_BF16, s));
    p = gemm_problem(pm, pn, pn, 1.f, R.Nb, R.ldn, R.QRb, R.ldn, 0.f, nullptr, 0,
                     out ? nullptr : U, out ? 0 : ldU, GF_D_F32);
  } else {
    p = gemm_problem(pm, pn, pn, 1.f, R.Mtil, R.ldn, st->QR.data, st->QR.ld, 0.f, nullptr, 0,
                     out ? nullptr : U, out ? 0 : ldU, GF_D_F32);
  }
  if (out) {
    p.Dt = U;
    p.lddt = ldU;
  }
  return gemm_add(gb, p, bb ? MAO_BF16 : MAO_F32, s);
}

mao_status foam_update(const mao_mat& W, RotBufs& R, const mao_foam_hparams* hp,
                       float* update_out, hipStream_t s) {
  const int m = (int)W.rows, n = (int)W.cols;
  int64_t ldU;
  float* U = foam_u(R, hp, n, update_out, ldU);
  return apply_update(view(W.data, W.ld), W.dtype, view(U, ldU), MAO_F32, m, n, 1, hp->lr,
                      hp->weight_decay, 1.f, nullptr, nullptr, view(nullptr, 0), s);
}

// ---- many matrices in one call: the QR refreshes grouped by size --------

struct QrJobRef {
  int mat;   // matrix index
  int side;  // 0: L (SOAP), 1: R
};

struct QrGroup {
  int n = 0;
  std::vector<QrJobRef> jobs;
  float* S = nullptr;
  float* E = nullptr;
  int* flags = nullptr;
  char* work = nullptr;
  char* eigh = nullptr;    // FOAM's eigendecomposition refresh: per-job workspaces
  int64_t ld = 0, sz = 0;  // leading dimension and per-job stride of S and E
  // bf16x3 refresh products: per-job operand splits (one region shared by
  // every group, so the groups' products run one group at a time)
  bf16_t* P3a = nullptr;
  bf16_t* P3b = nullptr;
  int64_t ld3 = 0, sz3 = 0;
};

// Carve per-matrix buffers, then the size groups (sorted by size): S and E of
// every job, FOAM's refresh flags, the QR workspaces. Deterministic in the
// shapes alone, so the size query and the step carve alike.
// fout: FOAM on the output side (buffers of the transposed problem, factor
// size m).
// gb: receives the pointer table of the grouped products (at most two
// products per matrix in a phase, five pointers each).
void carve_many(Carver& c, int count, const mao_mat* W, bool soap, std::vector<RotBufs>& R,
                std::vector<QrGroup>& groups, bool fout, GemmBatch* gb, const CarveOpt& o) {
  const bool eigh = o.eigh;
  R.assign(count, RotBufs{});
  std::vector<std::pair<int, QrJobRef>> all;
  for (int i = 0; i < count; ++i) {
    const int m = (int)W[i].rows, n = (int)W[i].cols;
    const bool t = !soap && fout;
    carve_rot(c, t ? n : m, t ? m : n, soap, true, R[i], false, o);
    if (soap) all.push_back({m, QrJobRef{i, 0}});
    all.push_back({t ? m : n, QrJobRef{i, 1}});
  }
  std::stable_sort(all.begin(), all.end(),
                   [](const std::pair<int, QrJobRef>& a, const std::pair<int, QrJobRef>& b) {
                     return a.first < b.first;
                   });
  groups.clear();
  for (const auto& e : all) {
    if (groups.empty() || groups.back().n != e.first) {
      groups.emplace_back();
      groups.back().n = e.first;
    }
    groups.back().jobs.push_back(e.second);
  }
  for (QrGroup& g : groups) {
    const int nj = (int)g.jobs.size();
    g.ld = ws_ld(g.n);
    g.sz = round_up((int64_t)g.n * g.ld, 64);
    g.S = c.take<float>((size_t)nj * g.sz);
    g.E = c.take<float>((size_t)nj * g.sz);
    g.flags = c.take<int>((size_t)nj);
    g.work = c.take<char>((size_t)nj * qr_work_stride(g.n));
    if (eigh) g.eigh = c.take<char>((size_t)nj * eigh_work_stride(g.n));
    for (int k = 0; k < nj; ++k) {
      RotBufs& r = R[g.jobs[k].mat];
      float* e = g.E + k * g.sz;
      if (g.jobs[k].side == 0) {
        r.EL = e;
      } else {
        r.ER = e;
        if (!soap) {
          r.S = g.S + k * g.sz;
          r.flag = g.flags + k;
        }
      }
    }
  }
  if (o.ref3) {
    size_t most = 0;
    for (QrGroup& g : groups) {
      g.ld3 = ws_ld(3 * split_width(g.n));
      g.sz3 = round_up((int64_t)g.n * g.ld3, 64);
      most = std::max(most, g.jobs.size() * (size_t)g.sz3);
    }
    bf16_t* a = c.take<bf16_t>(most);
    bf16_t* b = c.take<bf16_t>(most);
    for (QrGroup& g : groups) {
      g.P3a = a;
      g.P3b = b;
    }
  }
  const int64_t cap = (int64_t)2 * 5 * count;
  const void** table = c.take<const void*>((size_t)cap);
  if (gb) {
    gb->table = table;
    gb->capacity = cap;
  }
}

size_t many_ws(int count, const mao_mat* W, bool soap, bool fout, const CarveOpt& o) {
  Carver c(nullptr);
  std::vector<RotBufs> R;
  std::vector<QrGroup> groups;
  carve_many(c, count, W, soap, R, groups, fout, nullptr, o);
  return c.used + 256;
}

constexpr int kMaxMany = 4096;

mao_status check_many(int32_t count, const mao_mat* W, const mao_mat* G, const void* st) {
  if (count < 1 || count > kMaxMany) MAO_FAIL(MAO_E_SHAPE, "count=%d outside 1..%d", count, kMaxMany);
  if (!W || !G || !st) MAO_FAIL(MAO_E_NULL, "W, G or state array is NULL");
  return MAO_OK;
}

// row blocks of the column pass of the rank-1 power iteration
int rank1_col_blocks(int64_t rows) { return (int)std::min<int64_t>(rows, 128); }

}  // namespace

extern "C" {

mao_status soap_step(mao_mat W, mao_mat G, const mao_soap_state* st, int64_t t,
                     const mao_soap_hparams* hp, void* workspace, size_t workspace_bytes,
                     float* update_out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MAO_TRY(check_soap_hp(hp));
  std::vector<Range> rr;
  MAO_TRY(validate_soap(W, G, st, t, update_out, rr));
  MAO_TRY(check_no_overlap(rr));
  const int m = (int)W.rows, n = (int)W.cols;
  MAO_TRY(check_workspace(workspace, workspace_bytes, soap_workspace_size(m, n, hp)));
  Carver c(workspace);
  RotBufs R;
  carve_rot(c, m, n, true, true, R, true, soap_opt(hp));
  MAO_TRY(soap_pre(W, G, st, R, hp, nullptr, s));
  // 3b. refresh: Q <- qr(F Q); S = (F Q)^T = Q^T F stored row-major
  if (soap_refresh(hp, t)) {
    const int64_t ldS = ws_ld(std::max(m, n));
    if (R.P3a)
      MAO_TRY(nt3_split(m, R.EL, R.ldm, (const float*)st->L.data, st->L.ld, R.S, ldS, R.P3a,
                        R.P3b, R.ld3p, s, nullptr));
    else
      MAO_TRY(nt32(m, m, m, R.EL, R.ldm, (const float*)st->L.data, st->L.ld, R.S, ldS, nullptr, 0, s));
    MAO_TRY(qr_core(R.S, ldS, m, R.EL, R.ldm, (float*)st->QL.data, st->QL.ld, R.qr, nullptr, s,
                    false, R.P3a != nullptr));
    if (R.P3a)
      MAO_TRY(nt3_split(n, R.ER, R.ldn, (const float*)st->R.data, st->R.ld, R.S, ldS, R.P3a,
                        R.P3b, R.ld3p, s, nullptr));
    else
      MAO_TRY(nt32(n, n, n, R.ER, R.ldn, (const float*)st->R.data, st->R.ld, R.S, ldS, nullptr, 0, s));
    MAO_TRY(qr_core(R.S, ldS, n, R.ER, R.ldn, (float*)st->QR.data, st->QR.ld, R.qr, nullptr, s,
                    false, R.P3a != nullptr));
  }
  for (int stage = 0; stage < kSoapPostStages; ++stage)
    MAO_TRY(soap_post(stage, W, G, st, R, t, hp, update_out, nullptr, s));
  return MAO_OK;
}

size_t soap_step_many_workspace_size(int32_t count, const mao_mat* W, const mao_soap_hparams* hp) {
  if (!hp || !W || count < 1 || count > kMaxMany) return 0;
  for (int i = 0; i < count; ++i)
    if (W[i].rows < 1 || W[i].cols < 1) return 0;
  return many_ws(count, W, true, false, soap_opt(hp));
}

mao_status soap_step_many(int32_t count, const mao_mat* W, const mao_mat* G,
                          const mao_soap_state* st, int64_t t, const mao_soap_hparams* hp,
                          void* workspace, size_t workspace_bytes, float* const* update_out,
                          void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MAO_TRY(check_soap_hp(hp));
  MAO_TRY(check_many(count, W, G, st));
  std::vector<Range> rr;
  for (int i = 0; i < count; ++i)
    MAO_TRY(validate_soap(W[i], G[i], &st[i], t, update_out ? update_out[i] : nullptr, rr));
  MAO_TRY(check_no_overlap(rr));
  const CarveOpt o = soap_opt(hp);
  MAO_TRY(check_workspace(workspace, workspace_bytes, many_ws(count, W, true, false, o)));
  Carver c(workspace);
  std::vector<RotBufs> R;
  std::vector<QrGroup> groups;
  GemmBatch gb;
  carve_many(c, count, W, true, R, groups, false, &gb, o);
  for (int i = 0; i < count; ++i) MAO_TRY(soap_pre(W[i], G[i], &st[i], R[i], hp, &gb, s));
  MAO_TRY(gemm_flush(gb, s));
  if (soap_refresh(hp, t)) {
    // the QR inputs S = E F of every job, grouped, before the batched QRs
    for (QrGroup& g : groups) {
      for (int k = 0; k < (int)g.jobs.size(); ++k) {
        const int i = g.jobs[k].mat;
        const mao_mat& F = g.jobs[k].side == 0 ? st[i].L : st[i].R;
        if (o.ref3)
          MAO_TRY(nt3_split(g.n, g.E + k * g.sz, g.ld, (const float*)F.data, F.ld, g.S + k * g.sz,
                            g.ld, g.P3a + k * g.sz3, g.P3b + k * g.sz3, g.ld3, s, &gb));
        else
          MAO_TRY(nt32(g.n, g.n, g.n, g.E + k * g.sz, g.ld, (const float*)F.data, F.ld,
                       g.S + k * g.sz, g.ld, nullptr, 0, s, nullptr, &gb));
      }
      // bf16x3: the groups share one region of operand splits
      if (o.ref3) MAO_TRY(gemm_flush(gb, s));
    }
    MAO_TRY(gemm_flush(gb, s));
    // every size group in one refresh: their panels share launches
    std::vector<std::vector<float*>> q(groups.size());
    std::vector<std::vector<int64_t>> ldq(groups.size());
    std::vector<QrBatch> batches(groups.size());
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const QrGroup& g = groups[gi];
      const int nj = (int)g.jobs.size();
      q[gi].resize(nj);
      ldq[gi].resize(nj);
      for (int k = 0; k < nj; ++k) {
        const int i = g.jobs[k].mat;
        const mao_mat& Q = g.jobs[k].side == 0 ? st[i].QL : st[i].QR;
        q[gi][k] = (float*)Q.data;
        ldq[gi][k] = Q.ld;
      }
      QrBatch& b = batches[gi];
      b.n = g.n;
      b.njob = nj;
      b.S = g.S;
      b.ldS = g.ld;
      b.sS = g.sz;
      b.E = g.E;
      b.ldE = g.ld;
      b.sE = g.sz;
      b.Q = q[gi].data();
      b.ldQ = ldq[gi].data();
      b.work = g.work;
      b.fact_bf16x3 = o.ref3;
    }
    MAO_TRY(qr_core_multi(batches.data(), (int)batches.size(), s));
  }
  for (int stage = 0; stage < kSoapPostStages; ++stage) {
    for (int i = 0; i < count; ++i)
      MAO_TRY(soap_post(stage, W[i], G[i], &st[i], R[i], t, hp,
                        update_out ? update_out[i] : nullptr, &gb, s));
    MAO_TRY(gemm_flush(gb, s));
  }
  return MAO_OK;
}

// ---------------------------------------------------------------------------

size_t foam_workspace_size(int64_t rows, int64_t cols, const mao_foam_hparams* hp) {
  if (!hp || rows < 1 || cols < 1) return 0;
  if (foam_eigh(hp) && (hp->side == MAO_FOAM_OUTPUT ? rows : cols) > kEighMaxN) return 0;
  Carver c(nullptr);
  RotBufs R;
  const bool out = foam_out(hp);
  carve_rot(c, (int)(out ? cols : rows), (int)(out ? rows : cols), false, true, R, true,
            foam_opt(hp));
  return c.used + 256;
}

mao_status foam_step(mao_mat W, mao_mat G, const mao_foam_state* st, int64_t t,
                     const mao_foam_hparams* hp, void* workspace, size_t workspace_bytes,
                     float* update_out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MAO_TRY(check_foam_hp(hp));
  std::vector<Range> rr;
  MAO_TRY(validate_foam(W, G, st, t, hp, update_out, rr));
  MAO_TRY(check_no_overlap(rr));
  const int m = (int)W.rows, n = (int)W.cols;
  const bool out = foam_out(hp);
  const int k = out ? m : n;
  MAO_TRY(check_workspace(workspace, workspace_bytes, foam_workspace_size(m, n, hp)));
  Carver c(workspace);
  RotBufs R;
  carve_rot(c, out ? n : m, out ? m : n, false, true, R, true, foam_opt(hp));
  MAO_TRY(foam_pre(W, G, st, R, hp, nullptr, s));
  for (int stage = 0; stage < 3; ++stage)
    MAO_TRY(foam_criterion(k, st, R, t, hp, stage, nullptr, s, R.P3a, R.P3b, R.ld3p));
  if (foam_checks(hp, t) && foam_eigh(hp)) {
    // D = Q^T R Q from the criterion, diagonalised in the current basis
    EighJob job;
    job.D = R.D;
    job.ldD = R.ldn;
    job.Q = (float*)st->QR.data;
    job.ldQ = st->QR.ld;
    job.E = R.ER;
    job.ldE = R.ldn;
    EighBatch eb;
    eb.n = k;
    eb.njob = 1;
    eb.jobs = &job;
    eb.pred = R.flag;
    eb.work = R.eigh;
    MAO_TRY(eigh_batched(eb, s));
  } else if (foam_checks(hp, t)) {
    MAO_TRY(qr_core(R.S, R.ldn, k, R.ER, R.ldn, (float*)st->QR.data, st->QR.ld, R.qr, R.flag, s,
                    false, R.P3a != nullptr));
  }
  MAO_TRY(foam_rotate(W, G, st, R, hp, nullptr, s));
  MAO_TRY(foam_precondition_back(W, st, R, t, hp, update_out, nullptr, s));
  return foam_update(W, R, hp, update_out, s);
}

size_t foam_step_many_workspace_size(int32_t count, const mao_mat* W, const mao_foam_hparams* hp) {
  if (!hp || !W || count < 1 || count > kMaxMany) return 0;
  for (int i = 0; i < count; ++i) {
    if (W[i].rows < 1 || W[i].cols < 1) return 0;
    if (foam_eigh(hp) && (foam_out(hp) ? W[i].rows : W[i].cols) > kEighMaxN) return 0;
  }
  return many_ws(count, W, false, foam_out(hp), foam_opt(hp));
}

mao_status foam_step_many(int32_t count, const mao_mat* W, const mao_mat* G,
                          const mao_foam_state* st, int64_t t, const mao_foam_hparams* hp,
                          void* workspace, size_t workspace_bytes, float* const* update_out,
                          void* stream) {
  hipStream_t s = (hipStream_t)stream;
  MAO_TRY(check_foam_hp(hp));
  MAO_TRY(check_many(count, W, G, st));
  std::vector<Range> rr;
  for (int i = 0; i < count; ++i)
    MAO_TRY(validate_foam(W[i], G[i], &st[i], t, hp, update_out ? update_out[i] : nullptr, rr));
  MAO_TRY(check_no_overlap(rr));
  const CarveOpt o = foam_opt(hp);
  MAO_TRY(check_workspace(workspace, workspace_bytes,
                          many_ws(count, W, false, foam_out(hp), o)));
  Carver c(workspace);
  std::vector<RotBufs> R;
  std::vector<QrGroup> groups;
  GemmBatch gb;
  carve_many(c, count, W, false, R, groups, foam_out(hp), &gb, o);
  // phases: every matrix's products of a phase go out as grouped launches
  for (int i = 0; i < count; ++i) MAO_TRY(foam_pre(W[i], G[i], &st[i], R[i], hp, &gb, s));
  MAO_TRY(gemm_flush(gb, s));
  for (int stage = 0; stage < 3; ++stage) {
    if (o.ref3 && stage < 2 && foam_checks(hp, t)) {
      // bf16x3: the groups share one region of operand splits
      for (QrGroup& g : groups) {
        for (int k = 0; k < (int)g.jobs.size(); ++k) {
          const int i = g.jobs[k].mat;
          MAO_TRY(foam_criterion(g.n, &st[i], R[i], t, hp, stage, &gb, s, g.P3a + k * g.sz3,
                                 g.P3b + k * g.sz3, g.ld3));
        }
        MAO_TRY(gemm_flush(gb, s));
      }
      continue;
    }
    for (int i = 0; i < count; ++i)
      MAO_TRY(foam_criterion((int)(foam_out(hp) ? W[i].rows : W[i].cols), &st[i], R[i], t, hp,
                             stage, &gb, s));
    MAO_TRY(gemm_flush(gb, s));
  }
  if (foam_checks(hp, t) && foam_eigh(hp)) {
    for (QrGroup& g : groups) {
      const int nj = (int)g.jobs.size();
      std::vector<EighJob> jobs(nj);
      for (int k = 0; k < nj; ++k) {
        const int i = g.jobs[k].mat;
        jobs[k].D = R[i].D;
        jobs[k].ldD = R[i].ldn;
        jobs[k].Q = (float*)st[i].QR.data;
        jobs[k].ldQ = st[i].QR.ld;
        jobs[k].E = g.E + k * g.sz;
        jobs[k].ldE = g.ld;
      }
      EighBatch eb;
      eb.n = g.n;
      eb.njob = nj;
      eb.jobs = jobs.data();
      eb.pred = g.flags;
      eb.spred = 1;
      eb.work = g.eigh;
      MAO_TRY(eigh_batched(eb, s));
    }
  } else if (foam_checks(hp, t)) {
    std::vector<std::vector<float*>> q(groups.size());
    std::vector<std::vector<int64_t>> ldq(groups.size());
    std::vector<QrBatch> batches(groups.size());
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const QrGroup& g = groups[gi];
      const int nj = (int)g.jobs.size();
      q[gi].resize(nj);
      ldq[gi].resize(nj);
      for (int k = 0; k < nj; ++k) {
        const int i = g.jobs[k].mat;
        q[gi][k] = (float*)st[i].QR.data;
        ldq[gi][k] = st[i].QR.ld;
      }
      QrBatch& b = batches[gi];
      b.n = g.n;
      b.njob = nj;
      b.S = g.S;
      b.ldS = g.ld;
      b.sS = g.sz;
      b.E = g.E;
      b.ldE = g.ld;
      b.sE = g.sz;
      b.Q = q[gi].data();
      b.ldQ = ldq[gi].data();
      b.pred = g.flags;
      b.spred = 1;
      b.work = g.work;
      b.fact_bf16x3 = o.ref3;
    }
    MAO_TRY(qr_core_multi(batches.data(), (int)batches.size(), s));
  }
  for (int i = 0; i < count; ++i) MAO_TRY(foam_rotate(W[i], G[i], &st[i], R[i], hp, &gb, s));
  MAO_TRY(gemm_flush(gb, s));
  for (int i = 0; i < count; ++i)
    MAO_TRY(foam_precondition_back(W[i], &st[i], R[i], t, hp, update_out ? update_out[i] : nullptr,
                                   &gb, s));
  MAO_TRY(gemm_flush(gb, s));
  for (int i = 0; i < count; ++i)
    MAO_TRY(foam_update(W[i], R[i], hp, update_out ? update_out[i] : nullptr, s));
  return MAO_OK;
}

// ---------------------------------------------------------------------------

mao_status adamw_step(void* w, int32_t w_dtype, const void* g, int32_t g_dtype, float* m, float* v,
                      int64_t n, int64_t t, float lr, float beta1, float beta2, float eps,
                      float weight_decay, float* update_out, void* stream) {
  if (!w || !g || !m || !v) MAO_FAIL(MAO_E_NULL, "w, g, m or v is NULL");
  if (n < 1) MAO_FAIL(MAO_E_SHAPE, "n=%lld", (long long)n);
  if (!dtype_ok(w_dtype) || !dtype_ok(g_dtype)) MAO_FAIL(MAO_E_DTYPE, "w or g dtype");
  if (t < 1) MAO_FAIL(MAO_E_HPARAM, "t=%lld must be >= 1", (long long)t);
  MAO_TRY(check_adam_hp(lr, beta1, beta2, eps, weight_decay));
  if (((uintptr_t)w | (uintptr_t)g | (uintptr_t)m | (uintptr_t)v | (uintptr_t)update_out) % 16 != 0)
    MAO_FAIL(MAO_E_LAYOUT, "buffers must be 16-byte aligned");
  std::vector<Range> rr = {Range{(uintptr_t)w, (uintptr_t)w + n * dtype_size(w_dtype)},
                           Range{(uintptr_t)g, (uintptr_t)g + n * dtype_size(g_dtype)},
                           Range{(uintptr_t)m, (uintptr_t)(m + n)},
                           Range{(uintptr_t)v, (uintptr_t)(v + n)}};
  if (update_out) rr.push_back(Range{(uintptr_t)update_out, (uintptr_t)(update_out + n)});
  MAO_TRY(check_no_overlap(rr));
  const float bc1 = (float)(1.0 - pow((double)beta1, (double)t));
  const float bc2 = (float)(1.0 - pow((double)beta2, (double)t));
  return adamw(w, w_dtype, g, g_dtype, m, v, n, lr, beta1, beta2, bc1, bc2, eps, weight_decay,
               update_out, (hipStream_t)stream);
}

mao_status mao_gemm_nt(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                       const void* B, int64_t ldb, int32_t in_dtype, float beta, const float* C0,
                       int64_t ldc0, float* D, int64_t ldd, int32_t mode, void* stream) {
  if (!A || !B || !D) MAO_FAIL(MAO_E_NULL, "A, B or D is NULL");
  if (M < 1 || N < 1 || K < 1 || M > (1 << 20) || N > (1 << 20) || K > (1 << 20)) MAO_FAIL(MAO_E_SHAPE, "M, N, K");
  if (!dtype_ok(in_dtype)) MAO_FAIL(MAO_E_DTYPE, "in_dtype=%d", in_dtype);
  if (mode & ~(MAO_GEMM_SYMMETRIC | MAO_GEMM_B_KMAJOR)) MAO_FAIL(MAO_E_HPARAM, "mode=%d", mode);
  const bool sym = (mode & MAO_GEMM_SYMMETRIC) != 0, bkm = (mode & MAO_GEMM_B_KMAJOR) != 0;
  if (sym && bkm) MAO_FAIL(MAO_E_UNSUPPORTED, "symmetric with a K x N operand B");
  if (bkm && in_dtype != MAO_BF16) MAO_FAIL(MAO_E_UNSUPPORTED, "a K x N operand B needs bf16 inputs");
  if (lda < K || ldb < (bkm ? N : K) || lda % 8 || ldb % 8 || ldd < N || ldd % 8 || (C0 && (ldc0 < N || ldc0 % 8)))
    MAO_FAIL(MAO_E_LAYOUT, "leading dimensions");
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)D | (uintptr_t)C0) % 16 != 0) MAO_FAIL(MAO_E_LAYOUT, "alignment");
  if (sym && (M != N || A != B || lda != ldb)) MAO_FAIL(MAO_E_SHAPE, "symmetric needs A == B and M == N");
  if (!finite(alpha) || !finite(beta)) MAO_FAIL(MAO_E_HPARAM, "alpha/beta");
  GemmProblem p = gemm_problem((int)M, (int)N, (int)K, alpha, A, lda, B, ldb, beta, C0, ldc0, D, ldd,
                               GF_D_F32 | GF_C0_F32 | (sym ? GF_SYRK : 0) | (bkm ? GF_B_KMAJOR : 0));
  return launch_gemm(in_dtype, &p, 1, (hipStream_t)stream);
}

size_t mao_eigh_workspace_size(int64_t n) {
  if (n < 1 || n > kEighMaxN) return 0;
  return eigh_work_stride((int)n) + 256;
}

mao_status mao_eigh(const float* F, int64_t ldf, float* Q, int64_t ldq, float* evals, float* info,
                    int64_t n, void* workspace, size_t workspace_bytes, void* stream) {
  if (n > kEighMaxN) MAO_FAIL(MAO_E_UNSUPPORTED, "n=%lld above %d", (long long)n, kEighMaxN);
  MAO_TRY(check_mat("F", F, n, n, ldf, MAO_F32, true));
  MAO_TRY(check_mat("Q", Q, n, n, ldq, MAO_F32, true));
  if (((uintptr_t)evals | (uintptr_t)info) % 4 != 0) MAO_FAIL(MAO_E_LAYOUT, "evals / info misaligned");
  std::vector<Range> rr = {mat_range(F, 1, n, n, ldf, 0, 4), mat_range(Q, 1, n, n, ldq, 0, 4)};
  if (evals) rr.push_back(Range{(uintptr_t)evals, (uintptr_t)(evals + n)});
  if (info) rr.push_back(Range{(uintptr_t)info, (uintptr_t)(info + kEighMaxSweeps + 1)});
  MAO_TRY(check_no_overlap(rr));
  MAO_TRY(check_workspace(workspace, workspace_bytes, mao_eigh_workspace_size(n)));
  hipStream_t s = (hipStream_t)stream;
  MAO_TRY(fill_identity(view(Q, ldq), (int)n, nullptr, s));
  EighJob job;
  job.D = F;
  job.ldD = ldf;
  job.Q = Q;
  job.ldQ = ldq;
  job.evals = evals;
  EighBatch eb;
  eb.n = (int)n;
  eb.njob = 1;
  eb.jobs = &job;
  eb.work = (char*)workspace;
  eb.info = info;
  return eigh_batched(eb, s);
}

size_t mao_qr_workspace_size(int64_t n) {
  if (n < 1 || n > (1 << 20)) return 0;
  const int64_t ld = ws_ld(n);
  Carver c(nullptr);
  c.take<float>((size_t)n * ld);
  c.take<float>((size_t)n * ld);
  carve_qr_work(c, (int)n);
  return c.used + 256;
}

mao_status mao_qr(const float* P, int64_t ldp, float* Q, int64_t ldq, int64_t n, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return mao_dbg_qr(P, ldp, Q, ldq, n, workspace, workspace_bytes, 0, stream);
}

mao_status mao_dbg_qr(const float* P, int64_t ldp, float* Q, int64_t ldq, int64_t n,
                      void* workspace, size_t workspace_bytes, int32_t flags, void* stream) {
  if (flags & ~(MAO_DBG_QR_ABORT_BARRIERS | MAO_DBG_QR_NO_FALLBACK))
    MAO_FAIL(MAO_E_HPARAM, "flags=%d", flags);
  MAO_TRY(check_mat("P", P, n, n, ldp, MAO_F32, true));
  MAO_TRY(check_mat("Q", Q, n, n, ldq, MAO_F32, true));
  std::vector<Range> rr = {mat_range(P, 1, n, n, ldp, 0, 4), mat_range(Q, 1, n, n, ldq, 0, 4)};
  MAO_TRY(check_no_overlap(rr));
  MAO_TRY(check_workspace(workspace, workspace_bytes, mao_qr_workspace_size(n)));
  hipStream_t s = (hipStream_t)stream;
  const int64_t ld = ws_ld(n);
  Carver c(workspace);
  float* S = c.take<float>((size_t)n * ld);
  float* E = c.take<float>((size_t)n * ld);
  QrWork w = carve_qr_work(c, (int)n);
  MAO_TRY(transpose(view((void*)P, ldp), view(S, ld), (int)n, (int)n, 1, MAO_F32, s));
  return qr_core(S, ld, (int)n, E, ld, Q, ldq, w, nullptr, s,
                 (flags & MAO_DBG_QR_ABORT_BARRIERS) != 0, false,
                 (flags & MAO_DBG_QR_NO_FALLBACK) != 0);
}

// ---- observability ---------------------------------------------------------

size_t mao_matrix_rms_workspace_size(mao_batch X) {
  if (X.count < 1 || X.rows < 1 || X.cols < 1 || X.rows > (1 << 20)) return 0;
  Carver c(nullptr);
  c.take<double>((size_t)X.count * obs_rowblocks(X.rows));
  return c.used + 256;
}

mao_status mao_matrix_rms(mao_batch X, float* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  MAO_TRY(check_batch("X", X, false));
  if (X.count > 65535) MAO_FAIL(MAO_E_SHAPE, "count=%lld above 65535", (long long)X.count);
  if (!out) MAO_FAIL(MAO_E_NULL, "out is NULL");
  if ((uintptr_t)out % 4) MAO_FAIL(MAO_E_LAYOUT, "out not 4-byte aligned");
  std::vector<Range> rr = {batch_range(X), Range{(uintptr_t)out, (uintptr_t)(out + X.count)}};
  MAO_TRY(check_no_overlap(rr));
  MAO_TRY(check_workspace(workspace, workspace_bytes, mao_matrix_rms_workspace_size(X)));
  hipStream_t s = (hipStream_t)stream;
  Carver c(workspace);
  const int nrb = obs_rowblocks(X.rows);
  double* part = c.take<double>((size_t)X.count * nrb);
  MAO_TRY(sumsq_partials(view(X.data, X.ld, X.count > 1 ? X.stride : 0), X.dtype, (int)X.rows,
                         (int)X.cols, (int)X.count, nrb, false, part, s));
  return finalize_rms(part, nrb, (int)X.count, (double)X.rows * (double)X.cols, out, s);
}

size_t mao_ns_residual_workspace_size(mao_batch O) {
  if (O.count < 1 || O.rows < 1 || O.cols < 1 || O.rows > (1 << 20) || O.cols > (1 << 20))
    return 0;
  const int64_t a = std::min(O.rows, O.cols), b = std::max(O.rows, O.cols);
  Carver c(nullptr);
  c.take<float>((size_t)O.count * a * ws_ld(a));
  if (O.rows > O.cols) c.take<float>((size_t)O.count * a * ws_ld(b));
  c.take<double>((size_t)O.count * obs_rowblocks(a));
  return c.used + 256;
}

mao_status mao_ns_residual(mao_batch O, float scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  MAO_TRY(check_batch("O", O, true));
  if (O.count > 65535) MAO_FAIL(MAO_E_SHAPE, "count=%lld above 65535", (long long)O.count);
  if (!out) MAO_FAIL(MAO_E_NULL, "out is NULL");
  if ((uintptr_t)out % 4) MAO_FAIL(MAO_E_LAYOUT, "out not 4-byte aligned");
  if (!finite(scale) || scale == 0.f) MAO_FAIL(MAO_E_HPARAM, "scale=%g", (double)scale);
  std::vector<Range> rr = {batch_range(O), Range{(uintptr_t)out, (uintptr_t)(out + O.count)}};
  MAO_TRY(check_no_overlap(rr));
  MAO_TRY(check_workspace(workspace, workspace_bytes, mao_ns_residual_workspace_size(O)));
  hipStream_t s = (hipStream_t)stream;
  const int rows = (int)O.rows, cols = (int)O.cols, cnt = (int)O.count;
  const bool tall = rows > cols;
  const int a = std::min(rows, cols), b = std::max(rows, cols);
  const int64_t lda = ws_ld(a), ldt = ws_ld(b);
  Carver c(workspace);
  float* A = c.take<float>((size_t)cnt * a * lda);
  const float* X = (const float*)O.data;
  int64_t ldx = O.ld, sx = cnt > 1 ? O.stride : 0;
  if (tall) {
    float* T = c.take<float>((size_t)cnt * a * ldt);
    MAO_TRY(transpose(view(O.data, O.ld, sx), view(T, ldt, (int64_t)a * ldt), rows, cols, cnt,
                      MAO_F32, s));
    X = T;
    ldx = ldt;
    sx = (int64_t)a * ldt;
  }
  const int nrb = obs_rowblocks(a);
  double* part = c.take<double>((size_t)cnt * nrb);
  // A = (scale X)(scale X)^T on the wide orientation, one batched launch
  GemmProblem p = gemm_problem(a, a, b, scale * scale, X, ldx, X, ldx, 0.f, nullptr, 0, A, lda,
                               GF_SYRK | GF_D_F32);
  p.batch = cnt;
  p.sA = p.sB = sx;
  p.sD = (int64_t)a * lda;
  MAO_TRY(launch_gemm(MAO_F32, &p, 1, s));
  MAO_TRY(sumsq_partials(view(A, lda, (int64_t)a * lda), MAO_F32, a, a, cnt, nrb, true, part, s));
  return finalize_rms(part, nrb, cnt, (double)a, out, s);
}

size_t mao_rayleigh_workspace_size(int64_t n) {
  if (n < 1 || n > (1 << 20)) return 0;
  Carver c(nullptr);
  c.take<float>((size_t)n * ws_ld(n));
  c.take<float>((size_t)n * ws_ld(n));
  return c.used + 256;
}

mao_status mao_rayleigh(mao_mat F, mao_mat Q, float* diag_out, float* kappa_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  MAO_TRY(check_mat("F", F.data, F.rows, F.cols, F.ld, F.dtype, true));
  MAO_TRY(check_mat("Q", Q.data, Q.rows, Q.cols, Q.ld, Q.dtype, true));
  const int64_t n = F.rows;
  if (F.cols != n || Q.rows != n || Q.cols != n) MAO_FAIL(MAO_E_SHAPE, "F and Q must be n x n");
  if (!diag_out) MAO_FAIL(MAO_E_NULL, "diag_out is NULL");
  if ((uintptr_t)diag_out % 4 || (uintptr_t)kappa_out % 4) MAO_FAIL(MAO_E_LAYOUT, "outputs not 4-byte aligned");
  std::vector<Range> rr = {mrange(F), mrange(Q), Range{(uintptr_t)diag_out, (uintptr_t)(diag_out + n)}};
  if (kappa_out) rr.push_back(Range{(uintptr_t)kappa_out, (uintptr_t)(kappa_out + 1)});
  MAO_TRY(check_no_overlap(rr));
  MAO_TRY(check_workspace(workspace, workspace_bytes, mao_rayleigh_workspace_size(n)));
  hipStream_t s = (hipStream_t)stream;
  const int64_t ld = ws_ld(n);
  Carver c(workspace);
  float* Qt = c.take<float>((size_t)n * ld);
  float* C = c.take<float>((size_t)n * ld);
  MAO_TRY(transpose(view(Q.data, Q.ld), view(Qt, ld), (int)n, (int)n, 1, MAO_F32, s));
  // C[i][k] = sum_j Q[j][i] F[k][j] = (F Q)[k][i]; d_i = sum_k C[i][k] Q[k][i]
  MAO_TRY(nt32((int)n, (int)n, (int)n, Qt, ld, (const float*)F.data, F.ld, C, ld, nullptr, 0, s));
  MAO_TRY(row_dots(view(C, ld), view(Qt, ld), (int)n, (int)n, diag_out, s));
  if (kappa_out) MAO_TRY(kappa_of(diag_out, (int)n, kappa_out, s));
  return MAO_OK;
}

size_t mao_rank1_share_workspace_size(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || rows > (1 << 20) || cols > (1 << 20)) return 0;
  Carver c(nullptr);
  c.take<float>((size_t)cols);
  c.take<float>((size_t)rows);
  c.take<float>((size_t)rank1_col_blocks(rows) * cols);
  c.take<double>((size_t)obs_rowblocks(rows));
  return c.used + 256;
}

mao_status mao_rank1_share(mao_mat V, int32_t iters, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  MAO_TRY(check_mat("V", V.data, V.rows, V.cols, V.ld, V.dtype, true));
  if (iters < 1 || iters > 1000) MAO_FAIL(MAO_E_HPARAM, "iters=%d outside 1..1000", iters);
  if (!out) MAO_FAIL(MAO_E_NULL, "out is NULL");
  if ((uintptr_t)out % 4) MAO_FAIL(MAO_E_LAYOUT, "out not 4-byte aligned");
  std::vector<Range> rr = {mrange(V), Range{(uintptr_t)out, (uintptr_t)(out + 1)}};
  MAO_TRY(check_no_overlap(rr));
  MAO_TRY(check_workspace(workspace, workspace_bytes, mao_rank1_share_workspace_size(V.rows, V.cols)));
  hipStream_t s = (hipStream_t)stream;
  const int m = (int)V.rows, n = (int)V.cols;
  Carver c(workspace);
  float* v = c.take<float>((size_t)n);
  float* y = c.take<float>((size_t)m);
  const int nrbc = rank1_col_blocks(m);
  float* part = c.take<float>((size_t)nrbc * n);
  const int nrb = obs_rowblocks(m);
  double* vpart = c.take<double>((size_t)nrb);
  const View Vv = view(V.data, V.ld);
  MAO_TRY(sumsq_partials(Vv, MAO_F32, m, n, 1, nrb, false, vpart, s));
  // power iteration on V^T V from the unit all-ones vector
  MAO_TRY(fill_unit(v, n, s));
  for (int it = 0; it < iters; ++it) {
    MAO_TRY(gemv_rows(Vv, m, n, v, y, s));
    MAO_TRY(gemv_cols(Vv, m, n, y, part, nrbc, v, s));
    MAO_TRY(normalize_vec(v, n, s));
  }
  MAO_TRY(gemv_rows(Vv, m, n, v, y, s));
  return share_of(y, m, vpart, nrb, out, s);
}

mao_status mao_basis_age(const float* aux, float* age, void* stream) {
  if (!aux || !age) MAO_FAIL(MAO_E_NULL, "aux or age is NULL");
  if ((uintptr_t)aux % 4 || (uintptr_t)age % 4) MAO_FAIL(MAO_E_LAYOUT, "not 4-byte aligned");
  std::vector<Range> rr = {Range{(uintptr_t)aux, (uintptr_t)(aux + 4)},
                           Range{(uintptr_t)age, (uintptr_t)(age + 1)}};
  MAO_TRY(check_no_overlap(rr));
  return basis_age(aux, age, (hipStream_t)stream);
}

}  // extern "C"
