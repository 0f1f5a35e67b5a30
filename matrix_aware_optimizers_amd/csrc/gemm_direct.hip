// Large contractions (the Newton-Schulz products in bf16, the SOAP / FOAM
// rotations and factor products in fp32) with operands streamed straight from
// memory into LDS.
//
// D[i][j] = alpha * sum_k A[i][k] * B(j, k) + beta * C0[i][j], fp32
// accumulation on v_mfma_f32_32x32x16_bf16 (bf16 inputs) or
// v_mfma_f32_32x32x2f32 (fp32 inputs). B is either N x K (rows K-contiguous,
// as A) or, for bf16, K x N (the Newton-Schulz product B X reads X this way,
// so no transposed copy of X is ever written).
//
// Workgroup tile 256 x 256, 4 wavefronts in 2 x 2, each wavefront 128 x 128
// (4 x 4 MFMA blocks, 256 fp32 accumulators per lane). K advances in slices of
// 64 bytes per row (32 bf16 or 16 fp32 elements); a 16-byte chunk feeds one
// bf16 MFMA or four fp32 MFMAs, so an fp32 slice carries eight times the
// matrix-core work of a bf16 one over the same loads. Slices go global -> LDS with global_load_lds_dwordx4 (no
// staging registers) into a ring of four LDS stages, each its own LDS object,
// which lets the wait on a slice be an exact vmcnt rather than a full drain.
// The operand fragments of the next 16-deep MFMA step are read from LDS while
// the current step's MFMAs run (software pipelining pinned with scheduling
// groups). A K-contiguous tile keeps 64 bytes per row per slice, its four
// 16-byte chunks XOR-permuted by row bits 1-3 so that the 16-byte reads of 16
// consecutive rows hit distinct banks. A K x N tile keeps 32 k-rows of 512
// bytes, chunk bits 2-3 XOR-permuted by k-row bits 0-1, and is read with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16): each group of 16 lanes
// turns a 4 x 16 block into 16 columns of four consecutive k. A partial last
// slice (K not a multiple of 32) goes through registers with zero fill.
//
// Rows (columns) beyond M or N read a clamped, valid row (chunk); they only
// feed outputs that are never stored.
//
// Tiled operands (tiled.hpp) are zero-padded to whole tiles: a slice is then
// copied with no clamping, every direct load reading 1 KB in one piece, and
// a K x N slice sits in LDS as 8 blocks of 32 k-rows x 64 bytes.
//
// Epilogue (epilogue.hpp). The tiled bf16 results between Newton-Schulz
// iterations, and interior tiles of fp32 results without C0, leave straight
// from the accumulators (a quad transpose across lanes, 8- or 16-byte
// stores, no LDS). Other interior tiles, and every other tile of a tiled D,
// go through LDS in two halves of 128 rows and are written as whole rows in
// 16- or 32-byte pieces (C0 blend, row scale, transposed copy or SYRK mirror
// on the way). Edge tiles of a row-major D use 32-row bands through LDS.
#include "epilogue.hpp"
#include "gemm.hpp"

namespace mao {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int TB = 256;          // tile rows and columns
constexpr int ROWB = 64;         // bytes per tile row per slice (32 bf16 or 16 fp32 of K)
constexpr int STAGE = 2 * TB * ROWB;  // A and B of one slice: 32 KB
constexpr int LPT = (TB * ROWB / 16) / 256;  // 16-byte loads per thread per operand = 4
constexpr int SLAB_LD = TB + 1;
constexpr int SLAB_BYTES = 32 * SLAB_LD * 4;  // 32 rows of the output tile

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ uint32_t u4_at(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// K x N operand B: a slice is 32 k-rows of 512 bytes (the tile's 256 columns);
// 16-byte chunk c of k-row r sits at chunk c ^ bkswz(r), so the transposing
// reads of four consecutive k-rows hit distinct banks.
constexpr int BKROW = TB * 2;
__device__ __forceinline__ int bkswz(int krow) { return (krow & 3) << 2; }
typedef short lds_v4i16_t __attribute__((ext_vector_type(4), address_space(3)));

// s_waitcnt vmcnt(n), expcnt and lgkmcnt unconstrained (gfx9 field layout:
// vmcnt low bits [3:0], high bits [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define MAO_VMCNT(n) ((((n) & 0xf)) | (0x7 << 4) | (0xf << 8) | ((((n) >> 4) & 0x3) << 14))
template <int N>
__device__ __forceinline__ void vm_wait_c() { __builtin_amdgcn_s_waitcnt(MAO_VMCNT(N)); }
#define vm_wait(n) vm_wait_c<(n)>()



// DIRECT: every problem of the launch takes the direct tiled epilogue (the
// launcher checks it), so the staged epilogue is not compiled in and its
// register demand does not shape the rest of the kernel.
template <typename TIn, bool BKM, bool T32, bool DIRECT = false>
__device__ __forceinline__ void gemm_dl_body(const GemmArgs& args) {
  static_assert(sizeof(TIn) == 2 || (!BKM && !T32), "K x N and tiled operands are bf16 only");
  static_assert(!DIRECT || T32, "direct-only launches are tiled");
  constexpr bool F32 = sizeof(TIn) == 4;
  constexpr int EPC = 16 / (int)sizeof(TIn);  // elements per 16-byte chunk
  constexpr int KS = ROWB / (int)sizeof(TIn);  // K elements per slice
  __shared__ __attribute__((aligned(16))) unsigned char st0[(T32 || STAGE > SLAB_BYTES) ? STAGE : SLAB_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st3[STAGE];
  // tiled kernels never use the 32-row slab, so a fifth stage fits in 160 KB
  __shared__ __attribute__((aligned(16))) unsigned char st4[T32 ? STAGE : 16];

  // ---- tile --------------------------------------------------------------
  int pi, local;
  xcd_tile(args, blockIdx.x, pi, local);
  const GemmProblem& P = args.p[pi];
  const int b = local / P.tiles_per_batch;
  if (P.pred != nullptr && P.pred[b * P.spred] == 0) return;
  local -= b * P.tiles_per_batch;
  int tm, tn;
  const bool syrk = (P.flags & GF_SYRK) != 0;
  if (syrk) {
    tm = (int)((sqrtf(8.f * (float)local + 1.f) - 1.f) * 0.5f);
    while (tm > 0 && tm * (tm + 1) / 2 > local) --tm;
    while ((tm + 1) * (tm + 2) / 2 <= local) ++tm;
    tn = local - tm * (tm + 1) / 2;
  } else {
    constexpr int G = 8;
    const int per_group = G * P.tiles_n;
    const int grp = local / per_group;
    const int first_m = grp * G;
    const int gsz = min(G, P.tiles_m - first_m);
    const int in = local - grp * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
  }
  const int m0 = tm * TB, n0 = tn * TB;
  const int M = P.M, N = P.N, K = P.K;
  const TIn* A = (const TIn*)P.A + (int64_t)b * P.sA;
  const TIn* B = (const TIn*)P.B + (int64_t)b * P.sB;
  if constexpr (!T32) {
    if (P.ptab != nullptr) {  // pointer-table batch (tiled launches never take one)
      A = (const TIn*)P.ptab[5 * (int64_t)b];
      B = (const TIn*)P.ptab[5 * (int64_t)b + 1];
    }
  }
  const int64_t lda = P.lda, ldb = P.ldb;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // Per-thread sources of its LPT direct loads per operand. A (and B when it
  // is N x K): load p covers 16-byte slot (p * 4 + wave) * 64 + lane of the
  // tile, i.e. row slot / 4, chunk slot % 4 (permuted by swz). B when it is
  // K x N: load p covers k-rows 8 p + 2 wave + lane / 32 of the slice, chunk
  // lane % 32 of the row's 512 bytes (permuted by bkswz); columns past the
  // edge re-read the last valid chunk.
  //
  // Tiled operands: load p of wave w copies half-block (p * 4 + w) of the
  // slice, 1 KB read whole: block (8 tm + q / 2, slice) of A (and of an N x K
  // B), block (slice, 8 tn + q / 2) of a K x N B.
  const TIn* asrc[LPT];
  const TIn* bsrc[LPT];
#pragma unroll
  for (int p = 0; p < LPT; ++p) {
    if constexpr (T32) {
      const int q = p * 4 + wave;
      const int64_t half = (q & 1) * 512 + lane * 8;
      asrc[p] = A + (int64_t)(tm * 8 + (q >> 1)) * (lda >> 5) * 1024 + half;
      if constexpr (BKM)
        bsrc[p] = B + (int64_t)(tn * 8 + (q >> 1)) * 1024 + half;
      else
        bsrc[p] = B + (int64_t)(tn * 8 + (q >> 1)) * (ldb >> 5) * 1024 + half;
      continue;
    }
    const int L = (p * 4 + wave) * 64 + lane;  // 16-byte slot in the operand tile
    const int row = L >> 2, slot = L & 3;
    const int ch = slot ^ swz(row);
    const int ra = min(m0 + row, M - 1);
    asrc[p] = A + (int64_t)ra * lda + ch * EPC;
    if constexpr (BKM) {
      const int kr = 8 * p + 2 * wave + (lane >> 5);
      const int lc = (lane & 31) ^ bkswz(kr);
      const int col = min(n0 + 8 * lc, (N - 1) & ~7);
      bsrc[p] = B + (int64_t)kr * ldb + col;
    } else {
      const int rb = min(n0 + row, N - 1);
      bsrc[p] = B + (int64_t)rb * ldb + ch * EPC;
    }
  }
  // K offset k0 (elements) of a slice: along rows of A (and of an N x K B),
  // down the rows of a K x N B. Tiled: the next block of the block row (1024
  // elements per 32 k), or the next block row of a K x N B (32 ldb).
  const int64_t astep = T32 ? 32 : 1;
  const int64_t bstep = BKM ? ldb : astep;
  auto issue = [&](unsigned char* stage, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < LPT; ++p)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(asrc[p] + (int64_t)k0 * astep),
                                       (lds_void_t*)(stage + (p * 4 + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int p = 0; p < LPT; ++p)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(bsrc[p] + (int64_t)k0 * bstep),
                                       (lds_void_t*)(stage + TB * ROWB + (p * 4 + wave) * 1024), 16,
                                       0, 0);
  };

  // MFMA operand reads. Sub-step s of a slice multiplies the K elements of
  // 16-byte chunk 2 h + s in lane half h (bf16: one 16-deep MFMA; fp32: four
  // 2-deep MFMAs, element e of every lane's chunk in the e-th), the same
  // permutation on both operands. A (and an N x K B): lane (h, r32) reads
  // chunk 2 h + s of its rows.
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int arow = wm * 128 + r32, brow = wn * 128 + r32;
  const int ga = swz(arow), gb = swz(brow);  // same for rows +32, +64, +96
  const int aoff0 = arow * ROWB + (((2 * h + 0) ^ ga) << 4);
  const int aoff1 = arow * ROWB + (((2 * h + 1) ^ ga) << 4);
  const int boff0 = TB * ROWB + brow * ROWB + (((2 * h + 0) ^ gb) << 4);
  const int boff1 = TB * ROWB + brow * ROWB + (((2 * h + 1) ^ gb) << 4);
  // K x N B: two transposing 8-byte reads per fragment. In each group of 16
  // lanes, lane i names k-row (i / 4) and columns 4 (i % 4) .. + 3 of the
  // group's 4 x 16 block and receives column i of it, four k in order.
  const int ti = lane & 15, tg = (lane >> 4) & 1;
  int bko[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (T32) {
      // tiled K x N slice in LDS: 8 blocks of 32 k-rows x 64 bytes; read
      // (sub-step j / 2, upper four k j % 2) of fragment 0, fragments J at
      // +2 KB. Four k-rows of one block span all 64 banks.
      const int krow = 16 * h + 8 * (j >> 1) + 4 * (j & 1) + (ti >> 2);
      const int chunk = (2 * tg + ((ti >> 1) & 1)) ^ t32_swz(krow);
      bko[j] = TB * ROWB + wn * 4 * 2048 + krow * 64 + (chunk << 4) + 8 * (ti & 1);
    } else {
      const int krow = 16 * h + (ti >> 2);
      const int chunk = wn * 16 + ((j * 4) ^ bkswz(krow)) + 2 * tg + ((ti >> 1) & 1);
      bko[j] = TB * ROWB + krow * BKROW + (chunk << 4) + 8 * (ti & 1);
    }
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // B fragment j of sub-step SUB from stage STG (either layout)
#define MAO_BFRAG(STG, SUB, J, DST)                                                          \
  if constexpr (BKM && T32) {                                                               \
    const uint2 lo_ = __builtin_bit_cast(                                                   \
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                     \
                   (lds_v4i16_t*)(STG + bko[2 * (SUB)] + (J) * 2048)));                     \
    const uint2 hi_ = __builtin_bit_cast(                                                   \
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                     \
                   (lds_v4i16_t*)(STG + bko[2 * (SUB) + 1] + (J) * 2048)));                 \
    DST = make_uint4(lo_.x, lo_.y, hi_.x, hi_.y);                                           \
  } else if constexpr (BKM) {                                                               \
    const unsigned char* q_ = STG + bko[J] + (SUB) * 8 * BKROW;                             \
    const uint2 lo_ = __builtin_bit_cast(                                                   \
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(q_)));                \
    const uint2 hi_ = __builtin_bit_cast(                                                   \
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(q_ + 4 * BKROW)));    \
    DST = make_uint4(lo_.x, lo_.y, hi_.x, hi_.y);                                           \
  } else {                                                                                  \
    DST = *(const uint4*)(STG + ((SUB) ? boff1 : boff0) + (J) * 32 * ROWB);                 \
  }
#define MAO_READ(STG, SUB, FA, FB)                                                          \
  {                                                                                         \
    const int ao_ = (SUB) ? aoff1 : aoff0;                                                  \
    FA[0] = *(const uint4*)(STG + ao_);                                                     \
    MAO_BFRAG(STG, SUB, 0, FB[0])                                                           \
    FA[1] = *(const uint4*)(STG + ao_ + 32 * ROWB);                                         \
    MAO_BFRAG(STG, SUB, 1, FB[1])                                                           \
    FA[2] = *(const uint4*)(STG + ao_ + 64 * ROWB);                                         \
    MAO_BFRAG(STG, SUB, 2, FB[2])                                                           \
    FA[3] = *(const uint4*)(STG + ao_ + 96 * ROWB);                                         \
    MAO_BFRAG(STG, SUB, 3, FB[3])                                                           \
  }
  // fp32: the four 2-deep steps of a sub-step run over all 16 blocks in turn,
  // so consecutive MFMAs never accumulate into the same block.
#define MAO_MF(FA, FB, I, J)                                                                \
  if constexpr (F32) {                                                                      \
    acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(u4_at(FA[I], e_)),     \
                                                     __uint_as_float(u4_at(FB[J], e_)),     \
                                                     acc[I][J], 0, 0, 0);                   \
  } else {                                                                                  \
    acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, FA[I]), \
                                                        __builtin_bit_cast(bf16x8_t, FB[J]), \
                                                        acc[I][J], 0, 0, 0);                \
  }
#define MAO_MFMA16(FA, FB)                                                                  \
  _Pragma("unroll") for (int e_ = 0; e_ < (F32 ? 4 : 1); ++e_) {                           \
  MAO_MF(FA, FB, 0, 0) MAO_MF(FA, FB, 0, 1) MAO_MF(FA, FB, 1, 0) MAO_MF(FA, FB, 1, 1)       \
  MAO_MF(FA, FB, 0, 2) MAO_MF(FA, FB, 1, 2) MAO_MF(FA, FB, 2, 0) MAO_MF(FA, FB, 2, 1)       \
  MAO_MF(FA, FB, 2, 2) MAO_MF(FA, FB, 0, 3) MAO_MF(FA, FB, 1, 3) MAO_MF(FA, FB, 2, 3)       \
  MAO_MF(FA, FB, 3, 0) MAO_MF(FA, FB, 3, 1) MAO_MF(FA, FB, 3, 2) MAO_MF(FA, FB, 3, 3)       \
  }
  // Instruction order inside a sub-step: an operand read (and, in the second
  // sub-step, a direct load) after each of the first MFMAs.
#define MAO_SCHED(NR, NV)                                                                   \
  {                                                                                         \
    _Pragma("unroll") for (int q_ = 0; q_ < (F32 ? 64 : 16); ++q_) {                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                    \
      if (q_ < (NV)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                     \
      if (q_ < (NR)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                     \
    }                                                                                       \
  }

  // ---- main loop over full slices: 4-stage ring, pipelined operand reads ----
  // Slice k sits in stage k % 4. Step k multiplies sub-step 0 from fragments
  // read during the previous step while it reads sub-step 1; it then waits
  // for slice k + 1 (slice k + 2, 8 loads per thread, may still be in
  // flight), and after the barrier -- which also certifies that every
  // wave is done with the stage of slice k - 1 -- refills that stage with
  // slice k + 3 and reads sub-step 0 of slice k + 1 under the MFMAs of
  // sub-step 1. Past the end the last slice is reloaded into a stage nobody
  // reads again, so the loop has no branches. The tiled kernels run a
  // 5-stage ring the same way: slice k + 4 is issued at step k and slices
  // k + 2 and k + 3 may be in flight at its wait, a step more of lead.
  const int nkf = T32 ? (K + KS - 1) / KS : K / KS;  // full slices (tiled: zero pad past K)
  uint4 fa0[4], fb0[4], fa1[4], fb1[4];
  constexpr int NST = T32 ? 5 : 4;  // ring stages
#define MAO_RING_STEP(CUR, NXT, REF, K)                                 \
  {                                                                     \
    MAO_READ(CUR, 1, fa1, fb1)                                          \
    MAO_MFMA16(fa0, fb0)                                                \
    MAO_SCHED(BKM ? 12 : 8, 0)                                          \
    __builtin_amdgcn_sched_barrier(0);                                  \
    vm_wait((NST - 3) * 2 * LPT);                                       \
    asm volatile("" ::: "memory");                                      \
    __builtin_amdgcn_s_barrier();                                       \
    asm volatile("" ::: "memory");                                      \
    issue(REF, min((K) + NST - 1, nkf - 1) * KS);                       \
    MAO_READ(NXT, 0, fa0, fb0)                                          \
    MAO_MFMA16(fa1, fb1)                                                \
    MAO_SCHED(BKM ? 12 : 8, 2 * LPT)                                    \
    __builtin_amdgcn_sched_barrier(0);                                  \
  }
  int kt = 0;
  if (NST == 5 && nkf > 0) {
    issue(st0, 0);
    issue(st1, min(1, nkf - 1) * KS);
    issue(st2, min(2, nkf - 1) * KS);
    issue(st3, min(3, nkf - 1) * KS);
    vm_wait(3 * 2 * LPT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    MAO_READ(st0, 0, fa0, fb0)
    __builtin_amdgcn_sched_barrier(0);
    for (; kt + 5 <= nkf; kt += 5) {
      MAO_RING_STEP(st0, st1, st4, kt)
      MAO_RING_STEP(st1, st2, st0, kt + 1)
      MAO_RING_STEP(st2, st3, st1, kt + 2)
      MAO_RING_STEP(st3, st4, st2, kt + 3)
      MAO_RING_STEP(st4, st0, st3, kt + 4)
    }
    const int r = nkf - kt;
    if (r > 0) MAO_RING_STEP(st0, st1, st4, kt)
    if (r > 1) MAO_RING_STEP(st1, st2, st0, kt + 1)
    if (r > 2) MAO_RING_STEP(st2, st3, st1, kt + 2)
    if (r > 3) MAO_RING_STEP(st3, st4, st2, kt + 3)
  } else if (nkf > 0) {
    issue(st0, 0);
    issue(st1, min(1, nkf - 1) * KS);
    issue(st2, min(2, nkf - 1) * KS);
    vm_wait(2 * 2 * LPT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    MAO_READ(st0, 0, fa0, fb0)
    __builtin_amdgcn_sched_barrier(0);
    for (; kt + 4 <= nkf; kt += 4) {
      MAO_RING_STEP(st0, st1, st3, kt)
      MAO_RING_STEP(st1, st2, st0, kt + 1)
      MAO_RING_STEP(st2, st3, st1, kt + 2)
      MAO_RING_STEP(st3, st0, st2, kt + 3)
    }
    const int r = nkf - kt;
    if (r > 0) MAO_RING_STEP(st0, st1, st3, kt)
    if (r > 1) MAO_RING_STEP(st1, st2, st0, kt + 1)
    if (r > 2) MAO_RING_STEP(st2, st3, st1, kt + 2)
  }
#undef MAO_RING_STEP

  // ---- partial last slice through registers (zero fill past K) ------------
  const int ktail = nkf * KS;
  if (!T32 && ktail < K) {
    vm_wait(0);
    asm volatile("" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int p = 0; p < LPT; ++p) {
      const int L = (p * 4 + wave) * 64 + lane;
      union U {
        uint4 v;
        TIn e[EPC];
      } ua, ub;
      ua.v = make_uint4(0, 0, 0, 0);
      ub.v = make_uint4(0, 0, 0, 0);
      {
        const int row = L >> 2, slot = L & 3;
        const int k = ktail + (slot ^ swz(row)) * EPC;
        if (m0 + row < M)
          for (int e = 0; e < EPC; ++e)
            if (k + e < K) ua.e[e] = A[(int64_t)(m0 + row) * lda + k + e];
        if constexpr (!BKM) {
          if (n0 + row < N)
            for (int e = 0; e < EPC; ++e)
              if (k + e < K) ub.e[e] = B[(int64_t)(n0 + row) * ldb + k + e];
        }
      }
      if constexpr (BKM) {
        const int kr = L >> 5;
        const int col = n0 + 8 * ((L & 31) ^ bkswz(kr));
        if (ktail + kr < K)
          for (int e = 0; e < 8; ++e)
            if (col + e < N) ub.e[e] = B[(int64_t)(ktail + kr) * ldb + col + e];
      }
      *(uint4*)(st0 + L * 16) = ua.v;
      *(uint4*)(st0 + TB * ROWB + L * 16) = ub.v;
    }
    __syncthreads();
    MAO_READ(st0, 0, fa0, fb0)
    MAO_MFMA16(fa0, fb0)
    MAO_READ(st0, 1, fa1, fb1)
    MAO_MFMA16(fa1, fb1)
  }
#undef MAO_READ
#undef MAO_BFRAG
#undef MAO_MF
#undef MAO_MFMA16
#undef MAO_SCHED
  vm_wait(0);
  asm volatile("" ::: "memory");
  __syncthreads();
  if constexpr (DIRECT) {
    // the accumulators stay in AGPRs, read block by block by the epilogue:
    // held in VGPRs all at once, they leave the epilogue's addresses nowhere
    // to live but scratch
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
  }

  // ---- epilogue through LDS, 32 rows of the tile at a time ------------------
  const bool diag = syrk && (tm == tn);
  const bool d32 = (P.flags & GF_D_F32) != 0;
  const bool c32 = (P.flags & GF_C0_F32) != 0;
  const int dsz = d32 ? 4 : 2, csz = c32 ? 4 : 2;
  void* D = P.D ? (void*)((char*)P.D + (int64_t)b * P.sD * dsz) : nullptr;
  void* Tt = syrk ? D : (P.Dt ? (void*)((char*)P.Dt + (int64_t)b * P.sDt * dsz) : nullptr);
  const int64_t ldt = syrk ? P.ldd : P.lddt;
  const void* C0 = P.C0 ? (const void*)((const char*)P.C0 + (int64_t)b * P.sC0 * csz) : nullptr;
  if constexpr (!T32) {
    if (P.ptab != nullptr) {
      const OpPtrs o = problem_operands(P, b, (int)sizeof(TIn), csz, dsz);
      D = o.D;
      Tt = syrk ? o.D : o.Dt;
      C0 = o.C0;
    }
  }
  const float alpha = P.alpha, beta = P.beta;
  const float* rs = P.row_scale ? P.row_scale + b * P.srs : nullptr;
  // A tiled D is written whole, pad included (the pad of every operand is
  // zero, so it stays zero); a row-major D or Dt stops at M x N.
  const bool dt32 = (P.flags & GF_D_T32) != 0;
  if constexpr (T32 && BKM) {  // the B X products between iterations
    if (DIRECT || (dt32 && !syrk && !d32 && C0 == nullptr && Tt == nullptr && rs == nullptr &&
                   P.dadd == 0.f && D != nullptr)) {
      if (alpha == 1.f)
        direct_epilogue_t32<true>(acc, m0, n0, alpha, (bf16_t*)D, P.ldd);
      else
        direct_epilogue_t32<false>(acc, m0, n0, alpha, (bf16_t*)D, P.ldd);
      return;
    }
  }
  if constexpr (T32 && !BKM) {  // the symmetric products X X^T and A A + b A + a I
    if (DIRECT || (syrk && dt32 && !d32 && rs == nullptr && D != nullptr &&
                   (C0 == nullptr || ((P.flags & GF_C0_T32) != 0 && !c32)))) {
      if (C0 == nullptr && alpha == 1.f)
        direct_epilogue_t32_syrk<false, true>(acc, m0, n0, diag, alpha, nullptr, 0, 0.f, P.dadd, M,
                                              (bf16_t*)D, P.ldd);
      else if (C0 == nullptr)
        direct_epilogue_t32_syrk<false, false>(acc, m0, n0, diag, alpha, nullptr, 0, 0.f, P.dadd,
                                               M, (bf16_t*)D, P.ldd);
      else
        direct_epilogue_t32_syrk<true, false>(acc, m0, n0, diag, alpha, (const bf16_t*)C0, P.ldc0,
                                              beta, P.dadd, M, (bf16_t*)D, P.ldd);
      return;
    }
  }
  if constexpr (!DIRECT) {
  if constexpr (!T32) {  // fp32 results of the SOAP / FOAM products
    if (d32 && m0 + TB <= M && n0 + TB <= N && C0 == nullptr && rs == nullptr &&
        (D != nullptr || Tt != nullptr)) {
      direct_epilogue_f32(acc, m0, n0, diag, alpha, (float*)D, P.ldd, (float*)Tt, ldt);
      return;
    }
  }
  if ((m0 + TB <= M && n0 + TB <= N) || (T32 && dt32)) {
    EpiArgs ea;
    ea.m0 = m0; ea.n0 = n0; ea.M = M; ea.N = N;
    ea.alpha = alpha; ea.beta = beta;
    ea.C0 = C0; ea.ldc0 = P.ldc0; ea.c32 = c32;
    ea.rs = rs;
    ea.D = D; ea.ldd = P.ldd; ea.d32 = d32;
    ea.Tt = Tt; ea.ldt = ldt;
    ea.diag = diag;
    ea.c_t32 = (P.flags & GF_C0_T32) != 0;
    ea.d_t32 = dt32;
    ea.t_t32 = syrk && dt32;
    ea.dadd = T32 ? P.dadd : 0.f;
    staged_epilogue<false, T32>(acc, (float*)st0, (float*)st1, (float*)st2, (float*)st3, ea);
    return;
  }
  if constexpr (T32) {
    EpiArgs ea;
    ea.m0 = m0; ea.n0 = n0; ea.M = M; ea.N = N;
    ea.alpha = alpha; ea.beta = beta;
    ea.C0 = C0; ea.ldc0 = P.ldc0; ea.c32 = c32;
    ea.rs = rs;
    ea.D = D; ea.ldd = P.ldd; ea.d32 = d32;
    ea.Tt = Tt; ea.ldt = ldt;
    ea.diag = diag;
    ea.c_t32 = (P.flags & GF_C0_T32) != 0;
    ea.dadd = P.dadd;
    staged_epilogue<true, true>(acc, (float*)st0, (float*)st1, (float*)st2, (float*)st3, ea);
    return;
  } else {
  float* slab = (float*)st0;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // band rows: wm == half, block i -> tile rows half*128 + i*32 + [0, 32)
      __syncthreads();
      if (wm == half) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int sr = 8 * (v >> 2) + 4 * h + (v & 3);
            const int sc = wn * 128 + j * 32 + r32;
            slab[sr * SLAB_LD + sc] = acc[i][j][v];
          }
      }
      __syncthreads();
      const int rbase = m0 + half * 128 + i * 32;
      // direct pass: thread -> 4 consecutive columns of rows sr, sr+4, ...
      const int c4 = (threadIdx.x & 63) * 4;
      const int gcol = n0 + c4;
      for (int sr = threadIdx.x >> 6; sr < 32; sr += 4) {
        const int grow = rbase + sr;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = alpha * slab[sr * SLAB_LD + c4 + e];
        if (grow < M) {
          const bool full = gcol + 3 < N;
          if (C0) {
            const int64_t off = (int64_t)grow * P.ldc0 + gcol;
            if (full && c32) {
              const float4 c = *(const float4*)((const float*)C0 + off);
              v[0] += beta * c.x; v[1] += beta * c.y; v[2] += beta * c.z; v[3] += beta * c.w;
            } else if (full) {
              const uint2 c = *(const uint2*)((const bf16_t*)C0 + off);
              v[0] += beta * bf16_to_f32((bf16_t)(c.x & 0xffff));
              v[1] += beta * bf16_to_f32((bf16_t)(c.x >> 16));
              v[2] += beta * bf16_to_f32((bf16_t)(c.y & 0xffff));
              v[3] += beta * bf16_to_f32((bf16_t)(c.y >> 16));
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (gcol + e < N) v[e] += beta * c0_load(C0, c32, off + e);
            }
          }
          if (rs) {
            const float sc = rs[grow];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= sc;
          }
          if (D) {
            const int64_t off = (int64_t)grow * P.ldd + gcol;
            if (full && !diag) {
              if (d32) {
                *(float4*)((float*)D + off) = make_float4(v[0], v[1], v[2], v[3]);
              } else {
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                *(uint2*)((bf16_t*)D + off) = pk;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (gcol + e < N && (!diag || grow >= gcol + e)) d_store(D, d32, off + e, v[e]);
            }
          }
        }
        if (Tt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) slab[sr * SLAB_LD + c4 + e] = v[e];
        }
      }
      if (Tt) {
        __syncthreads();
        const int sr4 = (threadIdx.x & 7) * 4;
        const int grow = rbase + sr4;
        for (int sc = threadIdx.x >> 3; sc < TB; sc += 32) {
          const int gc = n0 + sc;
          if (gc >= N || grow >= M) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = slab[(sr4 + e) * SLAB_LD + sc];
          const int64_t off = (int64_t)gc * ldt + grow;
          if (!diag && grow + 3 < M) {
            if (d32) {
              *(float4*)((float*)Tt + off) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              uint2 pk;
              pk.x = pack_bf16x2(v[0], v[1]);
              pk.y = pack_bf16x2(v[2], v[3]);
              *(uint2*)((bf16_t*)Tt + off) = pk;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (grow + e < M && (!diag || grow + e > gc)) d_store(Tt, d32, off + e, v[e]);
          }
        }
      }
    }
  }
  }  // !T32
  }  // !DIRECT
}

template <bool BKM, bool T32, bool DIRECT = false>
__global__ __launch_bounds__(256) void gemm_bf16_dl_kernel(GemmArgs args) {
  gemm_dl_body<bf16_t, BKM, T32, DIRECT>(args);
}

__global__ __launch_bounds__(256) void gemm_f32_dl_kernel(GemmArgs args) {
  gemm_dl_body<float, false, false>(args);
}

}  // namespace

mao_status launch_gemm_f32_direct(GemmArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_f32_dl_kernel, dim3(args.total_tiles), dim3(256), 0, stream, args);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status launch_gemm_bf16_direct(GemmArgs& args, hipStream_t stream) {
  const bool bkm = (args.p[0].flags & GF_B_KMAJOR) != 0, t32 = (args.p[0].flags & GF_T32) != 0;
  const dim3 grid(args.total_tiles), block(256);
  // every problem's result leaves by the direct tiled epilogue: the
  // Newton-Schulz products between iterations (the kernel's own test, per
  // problem)
  bool direct = t32;
  for (int i = 0; i < args.nprob && direct; ++i) {
    const GemmProblem& p = args.p[i];
    const bool syrk = (p.flags & GF_SYRK) != 0;
    direct = (p.flags & GF_D_T32) != 0 && (p.flags & GF_D_F32) == 0 && p.row_scale == nullptr &&
             p.D != nullptr;
    if (bkm)
      direct = direct && !syrk && p.C0 == nullptr && p.Dt == nullptr && p.dadd == 0.f;
    else
      direct = direct && syrk &&
               (p.C0 == nullptr || ((p.flags & GF_C0_T32) != 0 && (p.flags & GF_C0_F32) == 0));
  }
  if (direct && bkm)
    hipLaunchKernelGGL((gemm_bf16_dl_kernel<true, true, true>), grid, block, 0, stream, args);
  else if (direct)
    hipLaunchKernelGGL((gemm_bf16_dl_kernel<false, true, true>), grid, block, 0, stream, args);
  else if (bkm && t32)
    hipLaunchKernelGGL((gemm_bf16_dl_kernel<true, true>), grid, block, 0, stream, args);
  else if (bkm)
    hipLaunchKernelGGL((gemm_bf16_dl_kernel<true, false>), grid, block, 0, stream, args);
  else if (t32)
    hipLaunchKernelGGL((gemm_bf16_dl_kernel<false, true>), grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL((gemm_bf16_dl_kernel<false, false>), grid, block, 0, stream, args);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

}  // namespace mao
