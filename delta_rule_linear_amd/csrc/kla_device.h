// Device helpers shared by the chunked kernels (kla_prefill.hip, kla_kda.hip,
// kla_ccq.hip, kla_bwd.hip): vector types, MFMA wrappers, the bf16 hi/lo
// split of an accumulator tile, LDS-only barriers, DPP lane movement and
// wave scans, range-checked buffer access, the XCD-aware workgroup order,
// the DPP forward-substitution step and the numbering of the off-diagonal
// Gram jobs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace kla {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int C = 64;             // chunk length
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int DVB = 16 * kWaves;  // dv columns per workgroup

__device__ inline f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Split4 {
  bf16x4 hi, lo;
};
struct Split8 {
  bf16x8 hi, lo;
};

// One accumulator tile as the B operand of a 16-deep MFMA (lane-group j
// holds contraction rows 4j..4j+3, exactly the tile's own rows), split into
// hi = bf16(x) (round to nearest even) + lo = bf16(x - hi).  The residual
// x - hi is exact in fp32; one v_dot2 of the packed hi pair with (-1, 0) or
// (0, -1) forms it without unpacking hi.
// The bf16 pairs (-1, 0) and (0, -1) as opaque scalar values: written by an
// s_mov the compiler cannot see through, so it never folds them into an
// inline constant (the inline constant -1.0 reads as the f32 bit pattern,
// i.e. the pair (0, -1), for packed bf16 operands).
__device__ inline bf16x2 sgpr_pair(uint32_t bits) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(bits));
  return __builtin_bit_cast(bf16x2, r);
}
__device__ inline Split4 split4(f32x4 c) {
  const bf16x2 m0 = sgpr_pair(0x0000BF80u), m1 = sgpr_pair(0xBF800000u);
  const bf16x2 h01 = __builtin_convertvector(__builtin_shufflevector(c, c, 0, 1), bf16x2);
  const bf16x2 h23 = __builtin_convertvector(__builtin_shufflevector(c, c, 2, 3), bf16x2);
  const f32x4 res = {__builtin_amdgcn_fdot2_f32_bf16(h01, m0, c[0], false),
                     __builtin_amdgcn_fdot2_f32_bf16(h01, m1, c[1], false),
                     __builtin_amdgcn_fdot2_f32_bf16(h23, m0, c[2], false),
                     __builtin_amdgcn_fdot2_f32_bf16(h23, m1, c[3], false)};
  Split4 r;
  r.hi = __builtin_shufflevector(h01, h23, 0, 1, 2, 3);
  r.lo = __builtin_convertvector(res, bf16x4);
  return r;
}
// Two tiles covering contraction rows [0,16) and [16,32) as the B operand of
// a 32-deep MFMA: element i of lane-group j holds row 4j+i (i<4) or
// 16+4j+(i-4) (i>=4).
__device__ inline Split8 join(const Split4 &a, const Split4 &b) {
  Split8 r;
  r.hi = __builtin_shufflevector(a.hi, b.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  r.lo = __builtin_shufflevector(a.lo, b.lo, 0, 1, 2, 3, 4, 5, 6, 7);
  return r;
}

// Column order of bf16 operand rows kept in LDS for the 32-deep MFMA (K and
// Q rows, the M planes' token columns, the per-channel-decay operands):
// within each 32-column block the 4-column groups sit in the order 0, 4, 1,
// 5, 2, 6, 3, 7.  A state
// fragment pair (rows 4j..4j+3 of two 16-row tiles) then meets its eight
// operand values in one 16-byte read, and a Gram tile, which contracts over
// this index on both sides, is unchanged.  pcol maps a logical column (a
// multiple of 4) to its place.
__device__ constexpr int pcol(int c) { return (c & ~31) + ((c & 15) >> 2) * 8 + ((c >> 4) & 1) * 4; }
static_assert(pcol(0) == 0 && pcol(4) == 8 && pcol(16) == 4 && pcol(20) == 12 && pcol(28) == 28 &&
                  pcol(44) == 56, "column order");

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also
// waits for every outstanding global load, which would expose the latency of
// the next chunk's prefetch at each barrier.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Hardware base-2 exponential and logarithm (v_exp_f32, v_log_f32, about
// 1 ulp).  Decay factors are 2^x with x <= 0; results below the normal range
// flush to zero, which is exact to the precision of the outputs.
__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float flog2(float x) { return __builtin_amdgcn_logf(x); }
// log2 of a decay rate in (0, 1]: rates below the smallest normal fp32
// number count as 2^-126 (what they multiply is below 2^-126 of its size
// either way), so the log stays finite even where the hardware log flushes
// subnormal inputs to zero.
__device__ inline float flog2_rate(float x) { return __builtin_amdgcn_logf(fmaxf(x, 0x1p-126f)); }

// Keep the instruction scheduler from moving code across this point; used to
// hold software-pipelined LDS loads ahead of the MFMAs that consume them.
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// DPP lane movement within 16-lane rows (gfx9 controls plus row_share).
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Same, but lanes whose source is outside the row (or rows masked off by
// ROWS) read zero.
template <int CTRL, int ROWS = 0xF>
__device__ inline float dpp0(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;       // quad_perm [1,0,3,2], [2,3,0,1]
constexpr int kHalfMirror = 0x141, kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane gets it.
template <int N>
__device__ inline float group_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (N == 8) {
    x += dpp<kHalfMirror>(x);
  } else {
    x += dpp<kRowRor4>(x);
    x += dpp<kRowRor8>(x);
  }
  if constexpr (N == 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline float wave_scan(float x) {
  x += dpp0<kRowShr1>(x);
  x += dpp0<kRowShr2>(x);
  x += dpp0<kRowShr4>(x);
  x += dpp0<kRowShr8>(x);
  x += dpp0<kRowBcast15, 0xA>(x);  // rows 1, 3 add the last lane of rows 0, 2
  x += dpp0<kRowBcast31, 0xC>(x);  // rows 2, 3 add lane 31
  return x;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// lane i receives element i%4 of the 8-byte chunks addressed by lanes
// 4e + i/4, e = 0..3.  With lane c addressing row (r0 + c/4), columns
// c0 + 4(c%4) .. +3 of a row-major tile, lane i gets column c0 + i of rows
// r0 .. r0+3: a transposed 4-element operand.
__device__ inline bf16x4 ld_tr(const bf16 *p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Range-checked buffer access: a load past the descriptor's byte range
// returns zero and a store past it is dropped, so ragged chunk tails and
// absent states need no branches (and no conservative waits on the memory
// counter around them).  Word 3 selects the 32-bit raw data format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)(uint32_t)b, 0x00020000);
}
__device__ inline uint4 buf_ld16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return uint4{v.x, v.y, v.z, v.w};
}
__device__ inline float buf_ld4(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ inline void buf_st16(rsrc_t r, uint32_t off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, 0);
}
// Non-temporal (cache policy nt): for outputs written once and not read back
// by the kernel, so they do not displace its inputs from the caches.
__device__ inline void buf_st16_nt(rsrc_t r, uint32_t off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, 2);
}
__device__ inline void buf_st4(rsrc_t r, uint32_t off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)off, 0, 0);
}

// XCD-aware workgroup order: consecutive logical ids land on one XCD so the
// dv-blocks of one (sequence, head) share that XCD's L2.  Bijective for any
// grid size, whatever the hardware dispatch order.
__device__ inline int64_t logical_block() {
  const int64_t G = gridDim.x, i = blockIdx.x;
  const int64_t q = G / 8, r = G % 8, x = i % 8, kx = i / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + kx;
}

// One column step of the 16x16 unit-lower-triangular substitution:
// x[r] += (-L[r][t]) x[t] for r > t, one v_fmac_f32_dpp per row whose first
// factor is broadcast from lane t of the 16-lane row.  The compiler adds no
// wait states in front of inline asm, so lc must not have been written by a
// VALU instruction within the two preceding wait states: callers load it
// from LDS or pass it through an s_nop (checked on the generated assembly by
// the test suite).
template <int T>
__device__ inline void solve_step(float (&x)[16], const float (&lc)[16]) {
#pragma unroll
  for (int r = T + 1; r < 16; ++r)
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(x[r]) : "v"(lc[r]), "v"(x[T]), "n"(T));
}
template <int... T>
__device__ inline void solve_steps(float (&x)[16], const float (&lc)[16],
                                   std::integer_sequence<int, T...>) {
  (solve_step<T>(x, lc), ...);
}

// Gram jobs of waves 1-3, numbered 0..15: jobs 0-5 are the K K^T blocks
// below the diagonal (-> -Ahat), in row order (1,0) (2,0) (2,1) (3,0) (3,1)
// (3,2); jobs 6-15 are the Q K^T blocks on or below the diagonal (-> M), in
// row order (0,0) (1,0) (1,1) (2,0) ... (3,3).  Decoded with scalar
// arithmetic from a wave-uniform job number.
struct Job {
  bool qk;
  int bi, bj;
};
__device__ inline Job job_of(int qj) {
  Job jb;
  jb.qk = qj >= 6;
  if (!jb.qk) {
    jb.bi = 1 + (qj >= 1) + (qj >= 3);
    jb.bj = qj - (jb.bi - 1) * jb.bi / 2;
  } else {
    const int p = qj - 6;
    jb.bi = (p >= 1) + (p >= 3) + (p >= 6);
    jb.bj = p - jb.bi * (jb.bi + 1) / 2;
  }
  return jb;
}

}  // namespace
}  // namespace kla
