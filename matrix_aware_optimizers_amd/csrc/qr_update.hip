// Fused panel step of the blocked Householder QR: one pass over the block
// that a 64-column panel updates applies the panel's reflector and projects
// the updated rows onto the next panel's Householder vectors,
//
//   C <- C - W Z^T              (C: M x L, W: M x nb, Z: L x nb)
//   Wn = C[:, 0:L] Vn^T         (Vn: nbn vectors as rows over C's columns)
//
// so the projection the next panel needs costs no second read of C (the
// separate route reads C once for the projection and once more, with the
// write, for the update: 12 bytes per element and panel against 8 here).
//
// Workgroup = 64 rows of C ("strip") and one of S contiguous column ranges
// ("split"; S raises the workgroup count when a panel's block has few
// strips), 4 wavefronts in 2 x 2; the workgroup walks its columns in chunks
// of 64. Per chunk: C's 64 x 64 block comes in by 16-byte loads into LDS,
// the update (W's fragments held in registers for the whole strip, Z's
// chunk in LDS as bf16 parts) turns it into D in place, D leaves by
// 16-byte stores, and the projection of D onto the chunk of Vn (both in LDS)
// accumulates in registers. The next chunk's Z and Vn, and C two chunks
// ahead, are loaded into registers while the current chunk's products run. Split s writes its
// partial projection into slice s of Wn; the consumer sums the slices (the
// next panel's call when it loads W, or a summing pass).
//
// Z and V come split already (qr_presplit_kernel, once per panel for all
// strips): only D is split inside the pass.
//
// The products run on bf16 MFMA in one of two arithmetics (QrPrec):
//  * bf16x3 (v_mfma_f32_32x32x16_bf16, fp32 accumulation): every fp32
//    operand x splits into hi = bf16(x) and lo = bf16(x - hi), A B^T = hi hi +
//    lo hi + hi lo (about 2^-17 relative per product). The factorisation
//    takes this when the power-iteration product it factors is itself
//    bf16x3: its rounding only perturbs the matrix factored, and the
//    reflectors stay exactly orthogonal;
//  * bf16x6, fp32-equivalent: x = hi + mid + lo exactly (three bf16 of 8
//    significant bits each cover fp32's 24), and the six products hh, hm, mh,
//    mm, hl, lh keep every term down to 2^-16 of the leading one; the
//    dropped ml, lm, ll are below 2^-24 relative. 6 bf16 products cost 6/16
//    of one fp32 product on the matrix cores. The explicit-Q accumulation
//    runs this way, and the factorisation when its input is an fp32
//    product.
//
// Optionally one more workgroup per job writes the first rows of Wn that
// come from identity rows of the next block (the explicit-Q accumulation:
// rows of E above the current panel are still rows of I, so their
// projection is a transposed copy of the vectors): Wt[c][i] = Vt[i][c] in
// slice 0, zero in the other slices.
#include <atomic>

#include "gemm.hpp"
#include "qr.hpp"

namespace mao {

namespace {

constexpr int FR = 64;       // rows per strip
constexpr int FC = 64;       // columns per chunk
constexpr int FK = 64;       // panel width (NB)
constexpr int LDF = FK + 4;  // LDS row pitch (floats)

__device__ __forceinline__ float4 ld4(const float* p, int k, int lim) {
  if (k + 4 <= lim) return *(const float4*)(p + k);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (k + e < lim) ? p[k + e] : 0.f;
  return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float comp(const float4& a, int e) {
  return e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w;
}

// Eight fp32 values (two float4) split into bf16 hi and lo fragments.
__device__ __forceinline__ void split8(const float4& x0, const float4& x1, uint4& hi, uint4& lo) {
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    const float r0 = v[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = v[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u);
    l[i] = pack_bf16x2(r0, r1);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Eight fp32 values split into bf16 hi, mid and lo fragments (x = hi + mid +
// lo exactly for normal x).
__device__ __forceinline__ void split8x3(const float4& x0, const float4& x1, uint4& hi, uint4& mid,
                                         uint4& lo) {
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    const float r0 = v[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = v[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u);
    m[i] = pack_bf16x2(r0, r1);
    l[i] = pack_bf16x2(r0 - __uint_as_float(m[i] << 16), r1 - __uint_as_float(m[i] & 0xffff0000u));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  mid = make_uint4(m[0], m[1], m[2], m[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ f32x16_t mfma_bf(const uint4& a, const uint4& b, f32x16_t acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// hh + mh + hm + mm + lh + hl, smallest terms first
__device__ __forceinline__ f32x16_t mfma6(const uint4& ah, const uint4& am, const uint4& al,
                                          const uint4& bh, const uint4& bm, const uint4& bl,
                                          f32x16_t acc) {
  acc = mfma_bf(al, bh, acc);
  acc = mfma_bf(ah, bl, acc);
  acc = mfma_bf(am, bm, acc);
  acc = mfma_bf(am, bh, acc);
  acc = mfma_bf(ah, bm, acc);
  return mfma_bf(ah, bh, acc);
}

__device__ __forceinline__ f32x16_t mfma3(const uint4& ah, const uint4& al, const uint4& bh,
                                          const uint4& bl, f32x16_t acc) {
  const bf16x8_t AH = __builtin_bit_cast(bf16x8_t, ah), AL = __builtin_bit_cast(bf16x8_t, al);
  const bf16x8_t BH = __builtin_bit_cast(bf16x8_t, bh), BL = __builtin_bit_cast(bf16x8_t, bl);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AH, BH, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AL, BH, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(AH, BL, acc, 0, 0, 0);
}

// LDS pitch of a bf16 part row (64 values + 8: the 16-byte operand reads of
// 8 consecutive rows fall on distinct banks)
constexpr int LDP = FK + 8;

template <int PREC>
__global__ __launch_bounds__(256, 2) void qr_fused_update_kernel(QrFusedArgs a) {
  constexpr bool X6 = PREC == kQrBf16x6;
  constexpr int NP = X6 ? 3 : 2;  // bf16 parts of a split operand
  __shared__ __attribute__((aligned(16))) bf16_t Zs[NP][FC * LDP];  // Z chunk: column x k
  __shared__ __attribute__((aligned(16))) bf16_t Vs[NP][FK * LDP];  // Vn chunk: vector x column
  __shared__ __attribute__((aligned(16))) float Ds[FR * LDF];  // C, then D, in place

  const int job = blockIdx.y;
  if (a.pred != nullptr && a.pred[job * a.spred] == 0) return;
  const int t = threadIdx.x;

  if ((int)blockIdx.x == a.strips * a.splits) {
    // identity rows: Wt[c][i] = Vt[i][c] (slice 0), zero in later slices
    const float* Vt = a.Vt + job * a.sV;
    float* Wt = a.Wt + job * a.sWn;
    for (int q = t; q < a.trows * FK; q += 256) {
      const int c = q / FK, i = q % FK;
      if (i >= a.nbn) continue;
      Wt[(int64_t)c * FK + i] = Vt[(int64_t)i * a.ldV + c];
      for (int sl = 1; sl < a.splits; ++sl) Wt[sl * a.wslice + (int64_t)c * FK + i] = 0.f;
    }
    return;
  }

  const int strip = blockIdx.x % a.strips, split = blockIdx.x / a.strips;
  const int r0 = strip * FR;
  const int M = a.M, L = a.L, nb = a.nb, nbn = a.nbn;
  const int nchunks = (L + FC - 1) / FC;
  const int per = (nchunks + a.splits - 1) / a.splits;
  const int ch0 = split * per, ch1 = min(nchunks, ch0 + per);
  float* C = a.C + job * a.sC;
  const float* W = a.W + job * a.sW;
  const bf16_t* Zp = a.Zp + job * a.sZp;
  const bf16_t* Vp = a.Vp + job * a.sVp;

  const int lane = t & 63, wave = t >> 6;
  const int rb = wave >> 1, cb = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  // this lane's 32 values of its row of W -- the sum of the producer's
  // slices, kept for every chunk: k = 16 s + 8 h .. + 7 for the 16-deep
  // steps s (lane half h), split into bf16 fragments.
  float wf[32];
  {
    const int row = r0 + rb * 32 + r32;
#pragma unroll
    for (int q = 0; q < 32; ++q) wf[q] = 0.f;
    if (row < M) {
      for (int sl = 0; sl < a.wslices_in; ++sl) {
        const float* wr = W + sl * a.wslice + (int64_t)row * FK;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int k = 16 * (q >> 1) + 8 * h + 4 * (q & 1);
          const float4 v = ld4(wr, k, nb);
          wf[4 * q + 0] += v.x;
          wf[4 * q + 1] += v.y;
          wf[4 * q + 2] += v.z;
          wf[4 * q + 3] += v.w;
        }
      }
    }
  }
  uint4 wh[4], wm[4], wl[4];
  {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float4 x0 = make_float4(wf[8 * st], wf[8 * st + 1], wf[8 * st + 2], wf[8 * st + 3]);
      const float4 x1 = make_float4(wf[8 * st + 4], wf[8 * st + 5], wf[8 * st + 6], wf[8 * st + 7]);
      if (X6)
        split8x3(x0, x1, wh[st], wm[st], wl[st]);
      else
        split8(x0, x1, wh[st], wl[st]);
    }
  }

  // chunk loads. C: thread -> 4-float piece (t % 16) of rows t / 16 + 16 i.
  // Z and Vn parts: thread -> 16-byte piece (t % 8) of rows t / 8 + 32 i of
  // every part (Z rows past L and Vn columns past L read as zero; the parts
  // are zero past nb and past Vn's columns). Z's and Vn's chunks are loaded
  // one chunk ahead, C's two chunks ahead (two register buffers used in
  // turn: the HBM read has two chunks' products to arrive in).
  const int pc = (t & 15) * 4, pr = t >> 4;
  const int qc = (t & 7) * 8, qr = t >> 3;
  uint4 zr[2 * NP], vr[2 * NP];
  float4 cr0[4], cr1[4];
  auto load_zv = [&](int c0) {
#pragma unroll
    for (int x = 0; x < NP; ++x)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = qr + 32 * i;  // Z row (chunk column) / vector index
        const int zc = c0 + row;
        uint4 z = make_uint4(0u, 0u, 0u, 0u), v = make_uint4(0u, 0u, 0u, 0u);
        if (zc < L) z = *(const uint4*)(Zp + x * a.zpart + (int64_t)zc * FK + qc);
        if (row < nbn && c0 + qc < L)
          v = *(const uint4*)(Vp + x * a.vpart + (int64_t)row * a.ldVp + c0 + qc);
        zr[2 * x + i] = z;
        vr[2 * x + i] = v;
      }
  };
  auto load_c = [&](int c0, float4 (&cr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cm = r0 + pr + 16 * i;
      cr[i] = cm < M ? ld4(C + (int64_t)cm * a.ldC + c0, pc, L - c0)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  f32x16_t accp;
#pragma unroll
  for (int v = 0; v < 16; ++v) accp[v] = 0.f;

  auto step = [&](int ch, float4 (&cr)[4]) __attribute__((always_inline)) {
    const int c0 = ch * FC;
    __syncthreads();  // the previous chunk's reads of Zs, Vs, Ds are done
#pragma unroll
    for (int x = 0; x < NP; ++x)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = qr + 32 * i;
        *(uint4*)&Zs[x][row * LDP + qc] = zr[2 * x + i];
        *(uint4*)&Vs[x][row * LDP + qc] = vr[2 * x + i];
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) *(float4*)&Ds[(pr + 16 * i) * LDF + pc] = cr[i];
    __syncthreads();
    if (ch + 1 < ch1) load_zv(c0 + FC);     // in flight during the products
    if (ch + 2 < ch1) load_c(c0 + 2 * FC, cr);

    // update: acc = W[rows of rb] Z[cols of cb]^T over k < 64
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    {
      const int zo = (cb * 32 + r32) * LDP + 8 * h;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint4 zh = *(const uint4*)&Zs[0][zo + 16 * st];
        const uint4 zl = *(const uint4*)&Zs[NP - 1][zo + 16 * st];
        if (X6) {
          const uint4 zm = *(const uint4*)&Zs[1][zo + 16 * st];
          acc = mfma6(wh[st], wm[st], wl[st], zh, zm, zl, acc);
        } else {
          acc = mfma3(wh[st], wl[st], zh, zl, acc);
        }
      }
    }
    // D = C - acc in place (each element read and written by one lane)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = rb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      float* d = &Ds[rl * LDF + cb * 32 + r32];
      *d = *d - acc[v];
    }
    __syncthreads();
    // D back to C in 16-byte pieces
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = pr + 16 * i, cm = r0 + row, col = c0 + pc;
      if (cm >= M || col >= L) continue;
      const float4 d = *(const float4*)&Ds[row * LDF + pc];
      float* dst = C + (int64_t)cm * a.ldC + col;
      if (col + 4 <= L) {
        *(float4*)dst = d;
      } else {
        for (int e = 0; col + e < L; ++e) dst[e] = comp(d, e);
      }
    }
    // projection: accp += D[rows of rb] Vn[vectors of cb]^T over the chunk
    if (nbn == 0) return;  // update only
    const float* db = Ds + (rb * 32 + r32) * LDF + 8 * h;
    const int vo = (cb * 32 + r32) * LDP + 8 * h;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float4 d0 = *(const float4*)(db + 16 * st), d1 = *(const float4*)(db + 16 * st + 4);
      const uint4 vh = *(const uint4*)&Vs[0][vo + 16 * st];
      const uint4 vl = *(const uint4*)&Vs[NP - 1][vo + 16 * st];
      if (X6) {
        const uint4 vm = *(const uint4*)&Vs[1][vo + 16 * st];
        uint4 dh, dm, dl;
        split8x3(d0, d1, dh, dm, dl);
        accp = mfma6(dh, dm, dl, vh, vm, vl, accp);
      } else {
        uint4 dh, dl;
        split8(d0, d1, dh, dl);
        accp = mfma3(dh, dl, vh, vl, accp);
      }
    }
  };

  if (ch0 < ch1) {
    load_zv(ch0 * FC);
    load_c(ch0 * FC, cr0);
  }
  if (ch0 + 1 < ch1) load_c((ch0 + 1) * FC, cr1);
#pragma unroll 1
  for (int ch = ch0; ch < ch1; ch += 2) {
    step(ch, cr0);
    if (ch + 1 < ch1) step(ch + 1, cr1);
  }

  // this split's partial Wn rows of the strip
  const int vec = cb * 32 + r32;
  if (vec < nbn) {
    float* Wn = a.Wn + job * a.sWn + split * a.wslice;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = r0 + rb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < M) Wn[(int64_t)row * FK + vec] = accp[v];
    }
  }
}

// Z (zrows x 64 at leading dimension 64, columns >= znb taken as zero) and
// V (vrows x vcols at ldV) of a panel split into their bf16 parts, 8 values
// per thread and part: Z's parts at row pitch 64, V's at ldVp (zero from
// vcols to the next multiple of 8).
__global__ __launch_bounds__(256) void qr_presplit_kernel(QrSplitArgs a) {
  const int job = blockIdx.y;
  if (a.pred != nullptr && a.pred[job * a.spred] == 0) return;
  const int64_t zq = (int64_t)a.zrows * 8;  // 8-value pieces of Z
  const int vc8 = (a.vcols + 7) / 8;
  const int64_t total = zq + (int64_t)a.vrows * vc8;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    float x[8];
    bf16_t* dst;
    int64_t part;
    if (q < zq) {
      const int row = (int)(q >> 3), c = (int)(q & 7) * 8;
      const float* src = a.Z + job * a.sZ + (int64_t)row * FK + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = c + e < a.znb ? src[e] : 0.f;
      dst = a.Zp + job * a.sZp + (int64_t)row * FK + c;
      part = a.zpart;
    } else {
      const int64_t v = q - zq;
      const int row = (int)(v / vc8), c = (int)(v % vc8) * 8;
      const float* src = a.V + job * a.sV + (int64_t)row * a.ldV + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = c + e < a.vcols ? src[e] : 0.f;
      dst = a.Vp + job * a.sVp + (int64_t)row * a.ldVp + c;
      part = a.vpart;
    }
    const float4 x0 = make_float4(x[0], x[1], x[2], x[3]), x1 = make_float4(x[4], x[5], x[6], x[7]);
    uint4 hi, mid, lo;
    if (a.parts == 3) {
      split8x3(x0, x1, hi, mid, lo);
      *(uint4*)(dst + part) = mid;
      *(uint4*)(dst + 2 * part) = lo;
    } else {
      split8(x0, x1, hi, lo);
      *(uint4*)(dst + part) = lo;
    }
    *(uint4*)dst = hi;
  }
}

}  // namespace

mao_status qr_presplit(const QrSplitArgs& a, int njob, hipStream_t stream) {
  if (njob <= 0) return MAO_OK;
  if (a.parts != 2 && a.parts != 3) return MAO_E_UNSUPPORTED;
  const int64_t total = (int64_t)a.zrows * 8 + (int64_t)a.vrows * ((a.vcols + 7) / 8);
  if (total <= 0) return MAO_OK;
  const int blocks = (int)std::min<int64_t>(1024, (total + 255) / 256);
  hipLaunchKernelGGL(qr_presplit_kernel, dim3(blocks, njob), dim3(256), 0, stream, a);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

// Cached per device; threads racing on the first call store the same value.
int qr_fused_slots() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int slots = cached[dev].load(std::memory_order_relaxed);
  if (slots == 0) {
    int cus = 0, b3 = 0, b6 = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b3, qr_fused_update_kernel<kQrBf16x3>, 256, 0) != hipSuccess) b3 = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b6, qr_fused_update_kernel<kQrBf16x6>, 256, 0) != hipSuccess) b6 = 1;
    slots = std::max(1, cus * std::max(1, std::min(b3, b6)));
    cached[dev].store(slots, std::memory_order_relaxed);
  }
  return slots;
}

mao_status qr_fused_update(const QrFusedArgs& args, int njob, hipStream_t stream) {
  QrFusedArgs a = args;
  if (njob <= 0 || a.M <= 0 || a.L <= 0) return MAO_OK;
  if (a.prec != kQrBf16x3 && a.prec != kQrBf16x6) return MAO_E_UNSUPPORTED;
  // the panel widths and the identity rows fit one 64-wide fragment
  if (a.nb < 1 || a.nb > FK || a.nbn < 0 || a.nbn > FK) return MAO_E_SHAPE;
  if (a.Wt != nullptr && (a.trows < 0 || a.trows > FK)) return MAO_E_SHAPE;
  // without a projection (nbn = 0) nothing is written per split, so any
  // number of column ranges may run side by side
  if (a.splits < 1 || (a.nbn > 0 && a.splits > kQrFusedMaxSplits) || a.wslices_in < 1 ||
      a.wslices_in > kQrFusedMaxSplits)
    return MAO_E_SHAPE;
  a.strips = (a.M + FR - 1) / FR;
  const int extra = a.Wt != nullptr ? 1 : 0;
  void* ev = nullptr;
  const bool timed = timing_on();
  if (timed) timing_record_begin(stream, &ev);
  const dim3 grid(a.strips * a.splits + extra, njob);
  if (a.prec == kQrBf16x3)
    hipLaunchKernelGGL(qr_fused_update_kernel<kQrBf16x3>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(qr_fused_update_kernel<kQrBf16x6>, grid, dim3(256), 0, stream, a);
  MAO_LAUNCH_CHECK();
  if (timed)
    timing_record_end(stream, ev, a.pred != nullptr ? TAG_GATED : TAG_QR_FUSED,
                      2.0 * a.M * (double)a.L * (a.nb + a.nbn) * njob);
  return MAO_OK;
}

}  // namespace mao
