// Chunkwise backward of the KLA prefill for gfx950.
//
// The KLA summary ("Resumo Tecnico: Atencao Linear Kaczmarz (KLA)", section
// "Implementacao") keeps Gated DeltaNet's chunk algorithm for training and
// changes only the step beta_t = eta_t / (|k_t|^2 + eps) (or beta_t = eta_t,
// the direct step).  This file computes the gradients of the prefill's
// outputs (o and the final state) with respect to q, k, v, alpha, eta and the
// initial state.
//
// Reverse recurrence.  With G_t the gradient of the state after token t plus
// the read's q_t dO_t^T, u_t = G_t^T k_t and dS_{t-1} = alpha_t (G_t - beta_t
// k_t u_t^T).  Inside a chunk of n tokens (gamma_t = alpha_1..alpha_t,
// Gam_ts = gamma_t / gamma_s for t >= s, B = Diag(beta), S the chunk-start
// state, Gend the gradient of the state after the chunk):
//   (I + StrictLower(Gam o K K^T) B) E = V - Diag(gamma) K S        residuals
//   (I + StrictUpper(Gam^T o K K^T) B) U = Diag(gamma_n/gamma) K Gend
//                                         + Mq^T dO,  Mq = Lower(Gam o Q K^T)
//   O        = Diag(gamma) Q S + Mq B E
//   dv       = B U,   dbeta_t = u_t . e_t
//   dk       = B (Diag(gamma_n/gamma) E Gend^T - Diag(gamma) U S^T + Z^T Q - W B K)
//              + Diag(dbeta o (beta^2 - 2 beta / (|k|^2 + eps))) K
//   dq       = Diag(gamma) dO S^T + Z B K
//   dS_start = gamma_n Gend + Q^T Diag(gamma) dO - K^T Diag(gamma beta) U
// with Z = Lower(Gam o dO E^T) and W the symmetric matrix W_ts = Gam_hl
// (u_h . e_l), h = max(t, s), l = min(t, s).  The direct step drops the
// -2 beta / (|k|^2 + eps) term.  The decay's gradient comes from a reverse
// running sum: c_t = alpha_t dalpha_t = c_{t+1} + dO_t . o_t - beta_t u_t . v_t,
// started at <Gend, S_end> at each chunk's end.
//
// Every quantity is linear in the state's columns (dv), so one workgroup of
// 8 waves (two per SIMD) takes one (sequence, head, DV columns of dv): the
// fp32 slices of S and Gend, K and Q of a chunk and the 64 x 64 planes fit
// in LDS.  With bf16 inputs K and Q stay bf16 in LDS and DV = 32; with fp32
// inputs DV = 16.  A first
// sweep runs the chunks forward and stores each chunk-start state slice in
// the workspace; the reverse sweep then takes the chunks from last to first.
// Products are fp32 MFMA (v_mfma_f32_16x16x4_f32), except dq and dk with bf16
// inputs, which run on the bf16 MFMA with every fp32 factor split hi/lo; the
// two triangular solves are 16 x 16 block substitutions whose diagonal blocks
// are inverted first, one wave per block, so the substitution itself is MFMA
// only.  The column slices' contributions to dq,
// dk, dbeta and c land in the workspace and a second kernel adds them in a
// fixed order (deterministic, no atomics) and finishes dk, deta, dalpha.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {
namespace {

constexpr int BW = 8;           // waves per workgroup (two per SIMD)
constexpr int BT = 64 * BW;     // threads per workgroup
constexpr int LDN = C + 4;      // row pitch of the 64 x 64 planes
constexpr int LDY = 20;         // row pitch of the 16 x 16 diagonal-block inverses

// State columns per workgroup and the LDS layout, per input type: bf16 K and
// Q are kept as bf16 (exact), which leaves room for 32 columns.
template <typename E, int D>
struct BwdCfg {
  static constexpr int DV = sizeof(E) == 2 ? 32 : 16;  // state columns per workgroup
  static constexpr int NCB = DV / 16;                  // 16-column blocks
  static constexpr int LDSL = DV + 4;                  // row pitch of the column-slice planes
  static constexpr int LDK = D + 16 / (int)sizeof(E);  // row pitch of K, Q (16-byte rows)
};

template <typename E, int D>
struct BwdSmem {
  using CF = BwdCfg<E, D>;
  alignas(16) E K[C * CF::LDK];
  alignas(16) E Q[C * CF::LDK];
  alignas(16) float Sc[D * CF::LDSL];  // chunk-start state, this workgroup's columns
  alignas(16) float Gd[D * CF::LDSL];  // gradient of the state after the chunk
  alignas(16) float Vs[C * CF::LDSL];
  alignas(16) float Ds[C * CF::LDSL];  // dO
  alignas(16) float Es[C * CF::LDSL];  // residuals e_t
  alignas(16) float Us[C * CF::LDSL];  // u_t
  alignas(16) float Am[C * LDN];   // lower: Gam o KK^T B; upper: its reverse twin; later W
  alignas(16) float Xm[C * LDN];   // Mq, later Z (lower, diagonal included)
  alignas(16) float Yl[4 * 16 * LDY];  // (I + L_bb)^-1, unit lower, per diagonal block
  alignas(16) float Yu[4 * 16 * LDY];  // (I + Lu_bb)^-1, unit upper
  alignas(16) float gl[C];    // cumulative log2 decay inside the chunk
  alignas(16) float gm[C];    // 2^gl
  alignas(16) float beta[C];
  float kk[C];
  float fc[C];    // per-row factor of the state update
  float scan[C];
  float la[C];    // log2 alpha of the chunk's rows (0 for padding or no decay)
  float eta[C];
  float tpart[CF::NCB][C];  // per 16-column block: sum_c dO[t][c] o[t][c]
  float red[BW];
};

__device__ inline float kf(float x) { return x; }
__device__ inline float kf(__bf16 x) { return static_cast<float>(x); }

struct Tok {
  int64_t bos;
  int L;
};

__device__ inline Tok seq_of(const BwdParams &p, int64_t s) {
  Tok t;
  t.bos = p.cu_seqlens ? (int64_t)p.cu_seqlens[s] : s * p.seq_len_dense;
  const int64_t eos = p.cu_seqlens ? (int64_t)p.cu_seqlens[s + 1] : t.bos + p.seq_len_dense;
  t.L = (int)(eos - t.bos);
  return t;
}

// 16x16 output tile, acc[i] = sum_k A(16 rows)[4j+i][k] B[k][c16] over
// K = 4 * steps, with the operands fetched by a(k) = A[c16][k] and
// b(k) = B[k][c16] (k the lane's own index 4 * step + j).
template <int STEPS, typename FA, typename FB>
__device__ __attribute__((always_inline)) inline f32x4 tile_mm(f32x4 acc, int k0, int j, FA a, FB b) {
#pragma unroll 4
  for (int st = 0; st < STEPS; ++st) {
    const int kx = k0 + 4 * st + j;
    acc = mma(a(kx), b(kx), acc);
  }
  return acc;
}
__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// A copy of a lane index that the compiler cannot hoist out of the chunk
// loop: addresses derived from it are recomputed where they are used rather
// than held (and spilled) across the loop, and every reload of a spill would
// wait for the chunk's prefetch and stores to drain.
__device__ inline int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
// Eight fp32 values as hi/lo bf16 halves of an MFMA operand.
__device__ inline Split8 split8f(const float (&x)[8]) {
  return join(split4(f32x4{x[0], x[1], x[2], x[3]}), split4(f32x4{x[4], x[5], x[6], x[7]}));
}

// Lower tile p (0..9) of a 4x4 block grid, in row order.
__device__ inline void lower_tile(int p, int &bt, int &bs) {
  bt = (p >= 1) + (p >= 3) + (p >= 6);
  bs = p - bt * (bt + 1) / 2;
}

// One chunk's operands in registers (16-byte segments), fetched a chunk
// ahead of their use with range-checked buffer loads: rows past the chunk's
// end read zero, so a ragged tail needs no branch.
template <typename E, int D>
struct Fetch {
  static constexpr int DV = BwdCfg<E, D>::DV;
  static constexpr int SEG_EL = 16 / sizeof(E);     // elements per segment
  static constexpr int SEG_ROW = D / SEG_EL;        // segments per K / Q row
  static constexpr int NKQ = C * SEG_ROW / BT;
  static constexpr int VSEG = DV / SEG_EL;          // segments per V row slice
  static constexpr int DSEG = DV / 4;               // segments per fp32 row slice
  static constexpr int NSSEG = D * DSEG;            // state-slice segments
  static constexpr int NSS = (NSSEG + BT - 1) / BT;
  static_assert(NKQ * BT == C * SEG_ROW, "tiling");
  static_assert(C * VSEG <= BT && C * DSEG <= BT, "slice tiling");
  uint4 k[NKQ], q[NKQ];
  uint4 v, d;
  uint4 s[NSS];
  float a, e;
};

template <typename E, int D>
__device__ inline void fetch(Fetch<E, D> &f, const BwdParams &p, int64_t t0, int n, int h,
                             int col0, const float *ckslot, bool rev, int tid_) {
  using F = Fetch<E, D>;
  constexpr int esz = sizeof(E);
  const int tid = fresh(tid_);
  const int64_t HD = (int64_t)p.H * D;
  const int64_t base = t0 * HD + (int64_t)h * D;
  const int64_t rows_kq = n > 0 ? ((int64_t)(n - 1) * HD + D) * esz : 0;
  const rsrc_t rk = make_rsrc(static_cast<const E *>(p.k) + base, rows_kq);
#pragma unroll
  for (int m = 0; m < F::NKQ; ++m) {
    const int sg = tid + BT * m, r = sg / F::SEG_ROW, cs = sg % F::SEG_ROW;
    f.k[m] = buf_ld16(rk, (uint32_t)(r * HD * esz + cs * 16));
  }
  if (rev) {
    const rsrc_t rq = make_rsrc(static_cast<const E *>(p.q) + base, rows_kq);
#pragma unroll
    for (int m = 0; m < F::NKQ; ++m) {
      const int sg = tid + BT * m, r = sg / F::SEG_ROW, cs = sg % F::SEG_ROW;
      f.q[m] = buf_ld16(rq, (uint32_t)(r * HD * esz + cs * 16));
    }
    const rsrc_t rd = make_rsrc(p.d_o + base + col0, n > 0 ? ((int64_t)(n - 1) * HD + F::DV) * 4 : 0);
    if (tid < C * F::DSEG)
      f.d = buf_ld16(rd, (uint32_t)((tid / F::DSEG) * HD * 4 + (tid % F::DSEG) * 16));
    const rsrc_t rs = make_rsrc(ckslot + col0, (int64_t)(D - 1) * D * 4 + F::DV * 4);
#pragma unroll
    for (int m = 0; m < F::NSS; ++m) {
      const int sg = tid + BT * m, r = sg / F::DSEG, cs = sg % F::DSEG;
      if (sg < F::NSSEG) f.s[m] = buf_ld16(rs, (uint32_t)((r * D + 4 * cs) * 4));
    }
  }
  const rsrc_t rv = make_rsrc(static_cast<const E *>(p.v) + base + col0,
                              n > 0 ? ((int64_t)(n - 1) * HD + F::DV) * esz : 0);
  if (tid < C * F::VSEG)
    f.v = buf_ld16(rv, (uint32_t)((tid / F::VSEG) * HD * esz + (tid % F::VSEG) * 16));
  if (tid < C) {
    const int64_t gb = t0 * p.H + h;
    const int64_t rows_s = n > 0 ? ((int64_t)(n - 1) * p.H + 1) * 4 : 0;
    f.e = buf_ld4(make_rsrc(p.eta + gb, rows_s), (uint32_t)(tid * p.H * 4));
    f.a = p.alpha ? buf_ld4(make_rsrc(p.alpha + gb, rows_s), (uint32_t)(tid * p.H * 4)) : 1.f;
  }
}

__device__ inline void cvt(const uint4 &u, __bf16, float (&x)[8]) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(b[e]);
}
__device__ inline void cvt(const uint4 &u, float, float (&x)[4]) {
  x[0] = __uint_as_float(u.x);
  x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z);
  x[3] = __uint_as_float(u.w);
}
__device__ inline void st4(float *dst, const float *x) {
  *reinterpret_cast<f32x4 *>(dst) = f32x4{x[0], x[1], x[2], x[3]};
}

// Registers -> LDS (K, Q in the input type, the rest fp32), with the row
// norms |k|^2 and the raw gates.
template <typename E, int D>
__device__ inline void commit(BwdSmem<E, D> &sm, const Fetch<E, D> &f, int n, bool rev, int tid_) {
  const int tid = fresh(tid_);
  using F = Fetch<E, D>;
  using CF = BwdCfg<E, D>;
  constexpr int LDK = CF::LDK, LDSL = CF::LDSL;
#pragma unroll
  for (int m = 0; m < F::NKQ; ++m) {
    const int sg = tid + BT * m, r = sg / F::SEG_ROW, cs = sg % F::SEG_ROW;
    float x[F::SEG_EL];
    cvt(f.k[m], E{}, x);
    float kk = 0.f;
#pragma unroll
    for (int e = 0; e < F::SEG_EL; ++e) kk = fmaf(x[e], x[e], kk);
    *reinterpret_cast<uint4 *>(&sm.K[r * LDK + cs * F::SEG_EL]) = f.k[m];
    kk = group_sum<F::SEG_ROW>(kk);  // the SEG_ROW lanes of row r hold its segments
    if (cs == 0) sm.kk[r] = kk;
    if (rev) *reinterpret_cast<uint4 *>(&sm.Q[r * LDK + cs * F::SEG_EL]) = f.q[m];
  }
  if (tid < C * F::VSEG) {
    float x[F::SEG_EL];
    cvt(f.v, E{}, x);
    const int r = tid / F::VSEG, cs = tid % F::VSEG;
#pragma unroll
    for (int e = 0; e < F::SEG_EL; e += 4) st4(&sm.Vs[r * LDSL + cs * F::SEG_EL + e], x + e);
  }
  if (rev) {
    float x[4];
    if (tid < C * F::DSEG) {
      cvt(f.d, float{}, x);
      st4(&sm.Ds[(tid / F::DSEG) * LDSL + (tid % F::DSEG) * 4], x);
    }
#pragma unroll
    for (int m = 0; m < F::NSS; ++m) {
      const int sg = tid + BT * m;
      if (sg < F::NSSEG) {
        cvt(f.s[m], float{}, x);
        st4(&sm.Sc[(sg / F::DSEG) * LDSL + (sg % F::DSEG) * 4], x);
      }
    }
  }
  if (tid < C) {
    sm.la[tid] = (tid < n && f.a != 1.f) ? flog2_rate(f.a) : 0.f;
    sm.eta[tid] = tid < n ? f.e : 0.f;
  }
}

// Row scalars from LDS: beta, the cumulative log2 decay and 2^gl (wave 0).
template <typename E, int D>
__device__ inline void row_scalars(BwdSmem<E, D> &sm, const BwdParams &p, int n, int tid) {
  if (tid < C) {
    const int r = tid;
    const float kk = sm.kk[r];
    const float eta = sm.eta[r];
    const float beta = r < n ? (p.beta_direct ? eta : eta / (kk + p.eps)) : 0.f;
    const float g = wave_scan(sm.la[r]);
    sm.beta[r] = beta;
    sm.gl[r] = g;
    sm.gm[r] = fexp2(g);
  }
}

// Stores one 16x16 tile of a lower-triangular 64 x 64 plane P (rows
// 16 bt + 4 j + i, column s = 16 bs + c16) scaled by the decay ratio
// Gam_ts = 2^(gl_t - gl_s): P[t][s] for t >= s and its mirror P[s][t] for
// t > s.  MODE 0: Lower(Gam o X) with zeros above; MODE 1: symmetric;
// MODE 2: Gam o K K^T B below the diagonal (times beta_s), its reverse twin
// above (times beta_t) and a zero diagonal.  The rows' decay logs come in
// one read and no element waits on another's loads; lanes with t < s store
// nothing (their clamped exponent cannot overflow).
template <int MODE>
__device__ __attribute__((always_inline)) inline void store_lower_tile(float *P, const float *gl, const float *beta,
                                                                      f32x4 acc, int bt, int bs, int j, int c16) {
  const int s = 16 * bs + c16, t0 = 16 * bt + 4 * j;
  const f32x4 glt = *reinterpret_cast<const f32x4 *>(&gl[t0]);
  const float gls = gl[s];
  f32x4 bt4 = {};
  float bss = 0.f;
  if constexpr (MODE == 2) {
    bt4 = *reinterpret_cast<const f32x4 *>(&beta[t0]);
    bss = beta[s];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + i;
    const float g = fexp2(fminf(glt[i] - gls, 0.f)) * acc[i];
    float dv = g, mv = 0.f;
    if constexpr (MODE == 1) mv = g;
    if constexpr (MODE == 2) {
      dv = t == s ? 0.f : g * bss;
      mv = g * bt4[i];
    }
    if (t >= s) P[t * LDN + s] = dv;
    if (t > s) P[s * LDN + t] = mv;
  }
}

// Am <- Gam o K K^T B below the diagonal and its reverse twin
// (Gam^T o K K^T B) above it; with_q: Xm <- Lower(Gam o Q K^T).  bf16 K and
// Q go to the bf16 MFMA (exact products, fp32 accumulation); fp32 inputs use
// the fp32 MFMA.
template <typename E, int D>
__device__ inline void gram(BwdSmem<E, D> &sm, bool with_q, int w, int j, int c16) {
  constexpr int LDK = BwdCfg<E, D>::LDK;
  const int jobs = with_q ? 20 : 10;
  for (int jb = w; jb < jobs; jb += BW) {
    const bool qk = jb >= 10;
    int bt, bs;
    lower_tile(qk ? jb - 10 : jb, bt, bs);
    const E *X = qk ? sm.Q : sm.K;
    f32x4 acc = zero4();
    if constexpr (sizeof(E) == 2) {
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        acc = mma(*reinterpret_cast<const bf16x8 *>(&X[(16 * bt + c16) * LDK + 32 * kb + 8 * j]),
                  *reinterpret_cast<const bf16x8 *>(&sm.K[(16 * bs + c16) * LDK + 32 * kb + 8 * j]),
                  acc);
    } else {
      acc = tile_mm<D / 4>(acc, 0, j, [&](int kx) { return X[(16 * bt + c16) * LDK + kx]; },
                           [&](int kx) { return sm.K[(16 * bs + c16) * LDK + kx]; });
    }
    if (qk)
      store_lower_tile<0>(sm.Xm, sm.gl, sm.beta, acc, bt, bs, j, c16);
    else
      store_lower_tile<2>(sm.Am, sm.gl, sm.beta, acc, bt, bs, j, c16);
  }
}

// A B for a 16-row block of a row-major input (K or Q) and one column of an
// fp32 row-major plane B, contracted over D: for fp32 inputs on the fp32
// MFMA; for bf16 inputs on the 16x16x32 bf16 MFMA, A exact (lane c16 of
// group j reads row c16 at k = 32 ks + 8 j .. +7, one 16-byte read) and B
// split hi/lo.  Result acc[i] is row 4 j + i of the block.
template <typename E, int D>
__device__ __attribute__((always_inline)) inline f32x4 rows_times_plane(const E *A, int lda, const float *B,
                                                                       int ldb, int j, int c16) {
  if constexpr (sizeof(E) == 2) {
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int k0 = 32 * ks + 8 * j;
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&A[c16 * lda + k0]);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = B[(k0 + e) * ldb];
      const Split8 b = split8f(x);
      acc = mma(a, b.hi, acc);
      acc = mma(a, b.lo, acc);
    }
    return acc;
  } else {
    return tile_mm<D / 4>(zero4(), 0, j, [&](int kx) { return kf(A[c16 * lda + kx]); },
                          [&](int kx) { return B[kx * ldb]; });
  }
}

// Es <- V - Diag(gamma) K S for tile `tile` (rows 16 (tile % 4), columns
// 16 (tile / 4) of the slice).
template <typename E, int D>
__device__ inline void residual_tile(BwdSmem<E, D> &sm, int tile, int j, int c16) {
  using CF = BwdCfg<E, D>;
  constexpr int LDK = CF::LDK, LDSL = CF::LDSL;
  const int bt = tile & 3, cc = 16 * (tile >> 2) + c16;
  const f32x4 acc = rows_times_plane<E, D>(&sm.K[16 * bt * LDK], LDK, &sm.Sc[cc], LDSL, j, c16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * bt + 4 * j + i;
    sm.Es[t * LDSL + cc] = sm.Vs[t * LDSL + cc] - sm.gm[t] * acc[i];
  }
}

// Inverses of the four unit triangular diagonal blocks of Am (lower: the
// strict lower parts; upper: the strict upper parts) into Y, one block per
// 16-lane row of the calling wave, by column substitution on the identity:
// lane t of a row holds column t of its block's triangle and column t of the
// result.  Each step broadcasts the pivot lane's triangle column across the
// row (v_fmac_f32_dpp row_newbcast, its negation a source modifier).  The
// triangle columns come straight from LDS, so no VALU write precedes their
// DPP reads.
template <int T, bool UPPER>
__device__ inline void inv_step(float (&x)[16], const float (&lc)[16]) {
#pragma unroll
  for (int r = UPPER ? 0 : T + 1; r < (UPPER ? T : 16); ++r)
    asm("v_fmac_f32_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(x[r]) : "v"(lc[r]), "v"(x[T]), "n"(T));
}
template <bool UPPER, int... T>
__device__ inline void inv_steps(float (&x)[16], const float (&lc)[16], std::integer_sequence<int, T...>) {
  if constexpr (UPPER)
    (inv_step<15 - T, true>(x, lc), ...);
  else
    (inv_step<T, false>(x, lc), ...);
}
template <bool UPPER>
__device__ inline void invert_blocks(const float *Am, float *Y, int l_) {
  const int l = fresh(l_), b = l >> 4, t = l & 15;
  const float *Lb = Am + 16 * b * LDN + 16 * b + t;
  float lc[16], x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) lc[r] = Lb[r * LDN];
  // a zero the compiler cannot hoist out of the caller's loop (the identity
  // would otherwise stay live in 16 registers across it)
  float zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = r == t ? 1.f : zero;
  inv_steps<UPPER>(x, lc, std::make_integer_sequence<int, 16>{});
#pragma unroll
  for (int r = 0; r < 16; ++r) Y[b * 16 * LDY + r * LDY + t] = x[r];
}

// Block substitution on 16 columns (from c0) of X (64 rows, pitch LDSL, in
// place) with the unit triangle of Am, the diagonal blocks applied through
// their inverses Y: for each block b (forward for the lower triangle,
// backward for the upper one)  X_b <- Y_b (X_b - sum_c Am_bc X_c).  One
// wave; MFMA only.  The solved blocks stay in registers, lane group j
// holding rows 4 j .. 4 j + 3 of each: that is the B operand of a step whose
// contraction index runs as 4 j + i, so the chain reads only the right-hand
// sides, Am and Y from LDS (the Am and Y rows by 16-byte reads), all of them
// independent of the chain.
template <bool UPPER, int LDSL>
__device__ inline void tri_solve_y(float *X, const float *Am, const float *Y, int c0, int j, int c16) {
  const int cc = c0 + c16;
  f32x4 xs[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[b][i] = X[(16 * b + 4 * j + i) * LDSL + cc];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int b = UPPER ? 3 - bb : bb;
    f32x4 acc = xs[b];
#pragma unroll
    for (int cb = 0; cb < bb; ++cb) {
      const int c = UPPER ? 3 - cb : cb;
      const f32x4 a = *reinterpret_cast<const f32x4 *>(&Am[(16 * b + c16) * LDN + 16 * c + 4 * j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = mma(-a[i], xs[c][i], acc);
    }
    const f32x4 y = *reinterpret_cast<const f32x4 *>(&Y[b * 16 * LDY + c16 * LDY + 4 * j]);
    f32x4 x = zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) x = mma(y[i], acc[i], x);
    xs[b] = x;
  }
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) X[(16 * b + 4 * j + i) * LDSL + cc] = xs[b][i];
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ inline f32x16 mma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// The column slice's contributions to dk and dq for rows 32 T .. 32 T + 31 and
// columns 32 I .. 32 I + 31 (v_mfma_f32_32x32x2_f32: lane l supplies row or
// column l % 32 at k = l / 32; result r of lane l is row 8 (r/4) + 4 (l/32)
// + r % 4, column l % 32):
//   dk = B (Diag(gamma_n/gamma) E Gend^T - Diag(gamma) U S^T + Z^T Q - W B K)
//   dq = Diag(gamma) dO S^T + Z B K
// The row scalings ride on the A operands, so each output has one
// accumulator, and the B K column reads serve both.
template <typename E, int D>
__device__ __attribute__((always_inline)) inline void dq_dk_tile(
    BwdSmem<E, D> &sm, int T, int I, int l, float glast, rsrc_t r_dq, rsrc_t r_dk, int64_t HD) {
  using CF = BwdCfg<E, D>;
  constexpr int LDK = CF::LDK, LDSL = CF::LDSL;
  const int r32 = l & 31, kh = l >> 5;
  const int ta = 32 * T + r32;  // this lane's A row
  const int ib = 32 * I + r32;  // this lane's B column
  const float fe = fexp2(glast - sm.gl[ta]), fg = sm.gm[ta];
  f32x16 ak = {}, aq = {};
#pragma unroll 2
  for (int st = 0; st < CF::DV / 2; ++st) {
    const int c = 2 * st + kh;
    const float sc = sm.Sc[ib * LDSL + c];
    ak = mma32(fe * sm.Es[ta * LDSL + c], sm.Gd[ib * LDSL + c], ak);
    ak = mma32(-fg * sm.Us[ta * LDSL + c], sc, ak);
    aq = mma32(fg * sm.Ds[ta * LDSL + c], sc, aq);
  }
  // Z^T Q over r >= 32 T (Z[r][t] = 0 for r < t)
  for (int g = T; g < 2; ++g) {
#pragma unroll 2
    for (int st = 16 * g; st < 16 * g + 16; ++st) {
      const int r = 2 * st + kh;
      ak = mma32(sm.Xm[r * LDN + ta], kf(sm.Q[r * LDK + ib]), ak);
    }
  }
  // - W B K over all s; Z B K over s < 32 (T + 1)
  for (int g = 0; g < 2; ++g) {
#pragma unroll 2
    for (int st = 16 * g; st < 16 * g + 16; ++st) {
      const int s2 = 2 * st + kh;
      const float kb = sm.beta[s2] * kf(sm.K[s2 * LDK + ib]);
      ak = mma32(-sm.Am[ta * LDN + s2], kb, ak);
      if (g <= T) aq = mma32(sm.Xm[ta * LDN + s2], kb, aq);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = 32 * T + 8 * (r >> 2) + 4 * kh + (r & 3);
    buf_st4(r_dk, (uint32_t)((t * HD + ib) * 4), sm.beta[t] * ak[r]);
    buf_st4(r_dq, (uint32_t)((t * HD + ib) * 4), aq[r]);
  }
}

// The same tile for bf16 inputs on v_mfma_f32_32x32x16_bf16 (lane l supplies
// contraction indices 16 s + 8 (l / 32) + 0..7 of its row or column); every
// fp32 factor enters split hi/lo, products as hi*hi + hi*lo + lo*hi (K and Q
// are bf16 and exact).  The contractions over rows take K and Q columns by
// transposing LDS reads: in each 16-lane group, lane i addresses row
// base + i / 4 at column group 4 (i % 4) and receives four rows of column i.
__device__ inline f32x16 mma32b(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mma32b3(const Split8 &a, const Split8 &b, f32x16 c) {
  c = mma32b(a.hi, b.hi, c);
  c = mma32b(a.hi, b.lo, c);
  return mma32b(a.lo, b.hi, c);
}
template <int D>
__device__ __attribute__((always_inline)) inline void dq_dk_tile_bf(
    BwdSmem<__bf16, D> &sm, int T, int I, int l, float glast, rsrc_t r_dq, rsrc_t r_dk, int64_t HD) {
  using CF = BwdCfg<__bf16, D>;
  constexpr int LDK = CF::LDK, LDSL = CF::LDSL, DV = CF::DV;
  const int r32 = l & 31, kh = l >> 5;
  const int ta = 32 * T + r32;  // this lane's A row
  const int ib = 32 * I + r32;  // this lane's B column
  const float fe = fexp2(glast - sm.gl[ta]), fg = sm.gm[ta];
  // transposing-read address of this lane for rows r0 + 8 kh.. of column block 32 I
  const int gi = l >> 4, li = l & 15;
  const int tr_row = 8 * (gi >> 1) + (li >> 2), tr_col = 32 * I + 16 * (gi & 1) + 4 * (li & 3);
  auto col8 = [&](const __bf16 *X, int r0) __attribute__((always_inline)) {  // X[r0 + 8 kh + e][ib]
    const bf16x4 a = ld_tr(&X[(r0 + tr_row) * LDK + tr_col]);
    const bf16x4 b = ld_tr(&X[(r0 + tr_row + 4) * LDK + tr_col]);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto ld8 = [&](const float *X, float f, float (&v)[8]) __attribute__((always_inline)) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(X);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(X + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = f * a[i];
      v[4 + i] = f * b[i];
    }
  };
  f32x16 ak = {}, aq = {};
  // over the slice's columns: E Gend^T and -U S^T (dk), dO S^T (dq); the S
  // split serves both
#pragma unroll 1
  for (int st = 0; st < DV / 16; ++st) {
    const int c0 = 16 * st + 8 * kh;
    float x[8], y[8];
    ld8(&sm.Es[ta * LDSL + c0], fe, x);
    ld8(&sm.Gd[ib * LDSL + c0], 1.f, y);
    ak = mma32b3(split8f(x), split8f(y), ak);
    ld8(&sm.Sc[ib * LDSL + c0], 1.f, y);
    const Split8 bs = split8f(y);
    ld8(&sm.Us[ta * LDSL + c0], -fg, x);
    ak = mma32b3(split8f(x), bs, ak);
    ld8(&sm.Ds[ta * LDSL + c0], fg, x);
    aq = mma32b3(split8f(x), bs, aq);
  }
  // Z^T Q over rows s >= 32 T: A[ta][s] = Xm[s][ta] (column reads), B = Q (exact)
  for (int st = 2 * T; st < 4; ++st) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sm.Xm[(16 * st + 8 * kh + e) * LDN + ta];
    const Split8 xs = split8f(x);
    const bf16x8 q8 = col8(sm.Q, 16 * st);
    ak = mma32b(xs.hi, q8, ak);
    ak = mma32b(xs.lo, q8, ak);
  }
  // - W B K over all s and Z B K over s < 32 (T + 1): beta_s joins the A rows
  // (Am, Xm), so the B operand is K itself (exact)
#pragma unroll 1
  for (int st = 0; st < 4; ++st) {
    const bf16x8 k8 = col8(sm.K, 16 * st);
    float be[8], x[8];
    ld8(&sm.beta[16 * st + 8 * kh], 1.f, be);
    ld8(&sm.Am[ta * LDN + 16 * st + 8 * kh], -1.f, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] *= be[i];
    const Split8 ws = split8f(x);
    ak = mma32b(ws.hi, k8, ak);
    ak = mma32b(ws.lo, k8, ak);
    if (st < 2 * (T + 1)) {
      ld8(&sm.Xm[ta * LDN + 16 * st + 8 * kh], 1.f, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] *= be[i];
      const Split8 zs = split8f(x);
      aq = mma32b(zs.hi, k8, aq);
      aq = mma32b(zs.lo, k8, aq);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = 32 * T + 8 * (r >> 2) + 4 * kh + (r & 3);
    buf_st4(r_dk, (uint32_t)((t * HD + ib) * 4), sm.beta[t] * ak[r]);
    buf_st4(r_dq, (uint32_t)((t * HD + ib) * 4), aq[r]);
  }
}

// The state-gradient tiles of a wave for bf16 inputs (16x16x32 bf16 MFMA):
// column block w & 1, row blocks (w >> 1) + 4 m.  The B operands
// gamma_t dO[t][c] and -gamma_t beta_t U[t][c] (lane group j holding
// t = 32 ks + 8 j + 0..7) are split hi/lo once and serve every row block;
// the A operands Q^T and K^T come exact by transposing reads.
template <int D, int NT>
__device__ __attribute__((always_inline)) inline void gend_tiles_bf(BwdSmem<__bf16, D> &sm, int w, int j,
                                                                   int c16, f32x4 (&gnew)[NT]) {
  using CF = BwdCfg<__bf16, D>;
  constexpr int LDK = CF::LDK, LDSL = CF::LDSL;
  const int cc = 16 * (w & 1) + c16;
  const float gn = sm.gm[C - 1];
#pragma unroll
  for (int m = 0; m < NT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) gnew[m][i] = gn * sm.Gd[(16 * ((w >> 1) + 4 * m) + 4 * j + i) * LDSL + cc];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int t0 = 32 * ks + 8 * j;
    float xd[8], xu[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = sm.gm[t0 + e];
      xd[e] = g * sm.Ds[(t0 + e) * LDSL + cc];
      xu[e] = -g * sm.beta[t0 + e] * sm.Us[(t0 + e) * LDSL + cc];
    }
    const Split8 bd = split8f(xd), bu = split8f(xu);
    // lane c16 of group j reads rows 32 ks + 8 j + c16 / 4 (and +4) at columns 16 ti + 4 (c16 % 4)..
    const int r = t0 + (c16 >> 2);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int co = 16 * ((w >> 1) + 4 * m) + 4 * (c16 & 3);
      const bf16x8 qa = __builtin_shufflevector(ld_tr(&sm.Q[r * LDK + co]), ld_tr(&sm.Q[(r + 4) * LDK + co]),
                                                0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 ka = __builtin_shufflevector(ld_tr(&sm.K[r * LDK + co]), ld_tr(&sm.K[(r + 4) * LDK + co]),
                                                0, 1, 2, 3, 4, 5, 6, 7);
      gnew[m] = mma(qa, bd.hi, gnew[m]);
      gnew[m] = mma(qa, bd.lo, gnew[m]);
      gnew[m] = mma(ka, bu.hi, gnew[m]);
      gnew[m] = mma(ka, bu.lo, gnew[m]);
    }
  }
}

// Tile m (0, 1) of a wave's share of the U right-hand side or read-out
// tiles (tile = bt + 4 cb), slot = wave - NCB, or -1.  With bf16 inputs the
// 8 tiles go to 6 waves; the two waves that take two tiles take the cheapest
// pairs: the U right-hand side's Mq^T dO part runs over 4 - bt row blocks,
// the read-out's Mq B E part over bt + 1.
template <int NCB>
__device__ inline int side_tile(bool readout, int slot, int m) {
  if constexpr (NCB == 2) {
    if (m == 0) return ((readout ? 0x627310 : 0x514023) >> (4 * slot)) & 15;
    return slot < 2 ? (readout ? 4 + slot : 7 - slot) : -1;
  } else {
    return m == 0 && slot < 4 * NCB ? slot : -1;
  }
}

template <typename E, int D>
__device__ inline float block_sum(BwdSmem<E, D> &sm, float x, int w, int l) {
  x = group_sum<32>(x);
  x += __shfl_xor(x, 32, 64);
  lds_barrier();
  if (l == 0) sm.red[w] = x;
  lds_barrier();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < BW; ++i) t += sm.red[i];
  return t;
}

template <typename E, int D>
__global__ __launch_bounds__(BT) void bwd_kernel(BwdParams p) {
  using CF = BwdCfg<E, D>;
  constexpr int LDK = CF::LDK, LDSL = CF::LDSL, DV = CF::DV, NCB = CF::NCB;
  constexpr int NS = D / DV;
  constexpr int DD = D * D;
  constexpr int NST = (D / 16) * NCB;  // 16x16 tiles of the state slice
  __shared__ BwdSmem<E, D> sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int j = l >> 4, c16 = l & 15;

  const int64_t lb = logical_block();
  const int sl = (int)(lb % NS);
  const int64_t sh = lb / NS;
  const int h = (int)(sh % p.H);
  const int64_t s = sh / p.H;
  const int col0 = sl * DV;
  const Tok sq = seq_of(p, s);
  const int nch = (sq.L + C - 1) / C;
  // checkpoint slots of this sequence: floor(bos / C) + s onwards (disjoint)
  float *ck = p.ws_ckpt + ((sq.bos / C + s) * p.H + h) * (int64_t)DD;
  const int64_t slot = (int64_t)p.H * DD;
  const int64_t TH = p.total_tok * p.H;
  using F = Fetch<E, D>;
  F f;

  // ---- forward sweep: chunk-start states -------------------------------
  // (skipped when the states-only prefill has written them, with the final
  // state in ws_fin)
  for (int idx = tid; idx < D * DV; idx += BT) {
    const int i = idx / DV, c = idx % DV;
    const float *src = p.ws_fin ? p.ws_fin : p.initial_state;
    sm.Sc[i * LDSL + c] = src ? src[sh * DD + i * D + col0 + c] : 0.f;
  }
  const int nfwd = p.ws_fin ? 0 : nch;
  if (nfwd > 0) fetch<E, D>(f, p, sq.bos, min(C, sq.L), h, col0, ck, false, tid);
  for (int ci = 0; ci < nfwd; ++ci) {
    const int n = min(C, sq.L - ci * C);
    lds_barrier();
    commit<E, D>(sm, f, n, false, tid);
#pragma unroll
    for (int m = 0; m < F::NSS; ++m) {
      const int sg = tid + BT * m, r = sg / F::DSEG, cs = sg % F::DSEG;
      if (sg < F::NSSEG)
        *reinterpret_cast<f32x4 *>(ck + ci * slot + (int64_t)r * D + col0 + 4 * cs) =
            *reinterpret_cast<const f32x4 *>(&sm.Sc[r * LDSL + 4 * cs]);
    }
    if (ci + 1 < nfwd)
      fetch<E, D>(f, p, sq.bos + (int64_t)(ci + 1) * C, min(C, sq.L - (ci + 1) * C), h, col0, ck,
                  false, tid);
    lds_barrier();
    row_scalars<E, D>(sm, p, n, tid);
    lds_barrier();
    gram<E, D>(sm, false, w, j, c16);
    if (tid < C) sm.fc[tid] = sm.beta[tid] * fexp2(sm.gl[C - 1] - sm.gl[tid]);
    lds_barrier();
    if (w == 0) invert_blocks<false>(sm.Am, sm.Yl, l);
    else if (w >= 4)
      for (int tile = w - 4; tile < 4 * NCB; tile += 4) residual_tile<E, D>(sm, tile, j, c16);
    lds_barrier();
    if (w < NCB) tri_solve_y<false, LDSL>(sm.Es, sm.Am, sm.Yl, 16 * w, j, c16);
    lds_barrier();
    // S <- gamma_n S + K^T Diag(beta gamma_n / gamma) E
    const float gn = sm.gm[C - 1];
    for (int tt = w; tt < NST; tt += BW) {
      const int ti = tt % (D / 16), cc = 16 * (tt / (D / 16)) + c16;
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = gn * sm.Sc[(16 * ti + 4 * j + i) * LDSL + cc];
      acc = tile_mm<C / 4>(acc, 0, j, [&](int kx) { return kf(sm.K[kx * LDK + 16 * ti + c16]); },
                           [&](int kx) { return sm.fc[kx] * sm.Es[kx * LDSL + cc]; });
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.Sc[(16 * ti + 4 * j + i) * LDSL + cc] = acc[i];
    }
  }
  // the checkpoints are read back below by the threads that wrote them
  __syncthreads();

  // ---- reverse sweep ----------------------------------------------------
  for (int idx = tid; idx < D * DV; idx += BT) {
    const int i = idx / DV, c = idx % DV;
    sm.Gd[i * LDSL + c] = p.d_final ? p.d_final[sh * DD + i * D + col0 + c] : 0.f;
  }
  if (nch > 0)
    fetch<E, D>(f, p, sq.bos + (int64_t)(nch - 1) * C, sq.L - (nch - 1) * C, h, col0,
                ck + (nch - 1) * slot, true, tid);
  lds_barrier();
  float cend;
  {
    float x = 0.f;
    for (int idx = tid; idx < D * DV; idx += BT) {
      const int i = idx / DV, c = idx % DV;
      x = fmaf(sm.Gd[i * LDSL + c], sm.Sc[i * LDSL + c], x);
    }
    cend = block_sum<E, D>(sm, x, w, l);
  }
  float *dqp = p.ws_dq + (int64_t)sl * TH * D;
  float *dkp = p.ws_dk + (int64_t)sl * TH * D;
  float *dbp = p.ws_db + (int64_t)sl * TH;
  float *cp = p.ws_c + (int64_t)sl * TH;

  const int64_t HD = (int64_t)p.H * D;
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int64_t t0 = sq.bos + (int64_t)ci * C;
    const int n = min(C, sq.L - ci * C);
    lds_barrier();
    commit<E, D>(sm, f, n, true, tid);
    if (ci > 0) fetch<E, D>(f, p, t0 - C, C, h, col0, ck + (ci - 1) * slot, true, tid);
    // range-checked stores: rows past the chunk's end are dropped
    const int64_t nrow = n - 1;
    const rsrc_t r_kk = make_rsrc(p.ws_kk + t0 * p.H + h, (nrow * p.H + 1) * 4);
    const rsrc_t r_db = make_rsrc(dbp + t0 * p.H + h, (nrow * p.H + 1) * 4);
    const rsrc_t r_c = make_rsrc(cp + t0 * p.H + h, (nrow * p.H + 1) * 4);
    const rsrc_t r_dv = make_rsrc(p.dv + t0 * HD + (int64_t)h * D + col0, (nrow * HD + DV) * 4);
    const rsrc_t r_dq = make_rsrc(dqp + t0 * HD + (int64_t)h * D, (nrow * HD + D) * 4);
    const rsrc_t r_dk = make_rsrc(dkp + t0 * HD + (int64_t)h * D, (nrow * HD + D) * 4);
    lds_barrier();
    row_scalars<E, D>(sm, p, n, tid);
    lds_barrier();
    if (sl == 0 && tid < C) buf_st4(r_kk, (uint32_t)(tid * p.H * 4), sm.kk[tid]);
    gram<E, D>(sm, true, w, j, c16);  // waves 0-3 take three Gram jobs, 4-7 two
    if (w >= 4)
      for (int tile = w - 4; tile < 4 * NCB; tile += 4) residual_tile<E, D>(sm, tile, j, c16);
    lds_barrier();
    if (w == 0) invert_blocks<false>(sm.Am, sm.Yl, l);
    else if (w == 4) invert_blocks<true>(sm.Am, sm.Yu, l);
    lds_barrier();
    const float glast = sm.gl[C - 1];
    if (w < NCB) {
      tri_solve_y<false, LDSL>(sm.Es, sm.Am, sm.Yl, 16 * w, j, c16);
    } else {
      // U right-hand side: Diag(gamma_n/gamma) K Gend + Mq^T dO
#pragma unroll 1
      for (int m = 0; m < 2; ++m) {
        const int tile = side_tile<NCB>(false, w - NCB, m);
        if (tile < 0) break;
        const int bt = tile & 3, cc = 16 * (tile >> 2) + c16;
        const f32x4 a1 = rows_times_plane<E, D>(&sm.K[16 * bt * LDK], LDK, &sm.Gd[cc], LDSL, j, c16);
        // Mq^T dO over rows s >= 16 bt, 16 rows (eight loads in flight) per step
        f32x4 a2 = zero4();
        for (int sb = bt; sb < 4; ++sb) {
          float xa[4], xb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kx = 16 * sb + 4 * j + i;
            xa[i] = sm.Xm[kx * LDN + 16 * bt + c16];
            xb[i] = sm.Ds[kx * LDSL + cc];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) a2 = mma(xa[i], xb[i], a2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * bt + 4 * j + i;
          sm.Us[t * LDSL + cc] = fexp2(glast - sm.gl[t]) * a1[i] + a2[i];
        }
      }
    }
    lds_barrier();
    if (w < NCB) {
      tri_solve_y<true, LDSL>(sm.Us, sm.Am, sm.Yu, 16 * w, j, c16);
    } else {
      // O = Diag(gamma) Q S + Mq B E, reduced at once to the rows' dO . o
#pragma unroll 1
      for (int m = 0; m < 2; ++m) {
        const int tile = side_tile<NCB>(true, w - NCB, m);
        if (tile < 0) break;
        const int bt = tile & 3, cb = tile >> 2, cc = 16 * cb + c16;
        const f32x4 a1 = rows_times_plane<E, D>(&sm.Q[16 * bt * LDK], LDK, &sm.Sc[cc], LDSL, j, c16);
        // Mq B E over rows s < 16 (bt + 1), 16 rows per step (Mq rows by 16-byte reads)
        f32x4 a2 = zero4();
        for (int sb = 0; sb <= bt; ++sb) {
          const f32x4 xa = *reinterpret_cast<const f32x4 *>(&sm.Xm[(16 * bt + c16) * LDN + 16 * sb + 4 * j]);
          const f32x4 be = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * sb + 4 * j]);
          float xb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) xb[i] = be[i] * sm.Es[(16 * sb + 4 * j + i) * LDSL + cc];
#pragma unroll
          for (int i = 0; i < 4; ++i) a2 = mma(xa[i], xb[i], a2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * bt + 4 * j + i;
          const float part = group_sum<16>(sm.Ds[t * LDSL + cc] * (sm.gm[t] * a1[i] + a2[i]));
          if (c16 == 0) sm.tpart[cb][t] = part;
        }
      }
    }
    lds_barrier();
    // per-row outputs: dv, the dbeta part and the decay running sum
    if (tid < C) {
      const int r = tid;
      const float b = sm.beta[r];
      float db = 0.f, term = 0.f;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) term += sm.tpart[cb][r];
#pragma unroll
      for (int c = 0; c < DV; ++c) {
        const float u = sm.Us[r * LDSL + c];
        db = fmaf(u, sm.Es[r * LDSL + c], db);
        term = fmaf(-b * u, sm.Vs[r * LDSL + c], term);
      }
      // suffix sum over rows r..63 (padded rows add zero)
      const float suf = wave_scan(__shfl(term, 63 - r, 64));
      sm.scan[63 - r] = suf;
      buf_st4(r_db, (uint32_t)(r * p.H * 4), db);
    }
    if (tid < C * F::DSEG) {
      const int r = tid / F::DSEG, cs = tid % F::DSEG;
      const float b = sm.beta[r];
      const f32x4 u = *reinterpret_cast<const f32x4 *>(&sm.Us[r * LDSL + 4 * cs]);
      buf_st16(r_dv, (uint32_t)(r * HD * 4 + cs * 16), f32x4{b * u[0], b * u[1], b * u[2], b * u[3]});
    }
    lds_barrier();
    if (tid < C) buf_st4(r_c, (uint32_t)(tid * p.H * 4), cend + sm.scan[tid]);
    // W (symmetric, from U E^T) into Am; Z = Lower(Gam o dO E^T) into Xm
    for (int jb = w; jb < 20; jb += BW) {
      const bool zq = jb >= 10;
      int bt, bs;
      lower_tile(zq ? jb - 10 : jb, bt, bs);
      const float *X = zq ? sm.Ds : sm.Us;
      // contraction over the slice's columns, lane group j taking columns
      // DV / 4 j .. +DV / 4 - 1 of both rows (16-byte reads, all in flight at once)
      f32x4 acc = zero4();
      {
        constexpr int NK = DV / 16;
        f32x4 a[NK], b[NK];
#pragma unroll
        for (int q = 0; q < NK; ++q) {
          a[q] = *reinterpret_cast<const f32x4 *>(&X[(16 * bt + c16) * LDSL + (DV / 4) * j + 4 * q]);
          b[q] = *reinterpret_cast<const f32x4 *>(&sm.Es[(16 * bs + c16) * LDSL + (DV / 4) * j + 4 * q]);
        }
#pragma unroll
        for (int q = 0; q < NK; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mma(a[q][e], b[q][e], acc);
      }
      if (zq)
        store_lower_tile<0>(sm.Xm, sm.gl, sm.beta, acc, bt, bs, j, c16);
      else
        store_lower_tile<1>(sm.Am, sm.gl, sm.beta, acc, bt, bs, j, c16);
    }
    lds_barrier();
    // dq and dk contributions of these columns, as 32 x 32 tiles: wave w takes
    // row block w & 1 and column block w >> 1 of both (D = 64: waves 0-3)
    if (w < D / 16) {
      if constexpr (sizeof(E) == 2)
        dq_dk_tile_bf<D>(sm, w & 1, w >> 1, l, glast, r_dq, r_dk, HD);
      else
        dq_dk_tile<E, D>(sm, w & 1, w >> 1, l, glast, r_dq, r_dk, HD);
    }
    // Gend <- gamma_n Gend + Q^T Diag(gamma) dO - K^T Diag(gamma beta) U
    constexpr int NT = (NST + BW - 1) / BW;  // state tiles per wave
    auto gtile = [&](int m, int &ti, int &cc) {
      if constexpr (sizeof(E) == 2) {
        ti = (w >> 1) + 4 * m;
        cc = 16 * (w & 1) + c16;
      } else {
        const int tt = w + BW * m;
        ti = tt % (D / 16);
        cc = 16 * (tt / (D / 16)) + c16;
      }
    };
    f32x4 gnew[NT];
    if constexpr (sizeof(E) == 2) {
      static_assert(NT * BW == NST, "bf16 state tiling");
      gend_tiles_bf<D, NT>(sm, w, j, c16, gnew);
    } else {
      const float gn = sm.gm[C - 1];
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        if (w + BW * m >= NST) break;
        int ti, cc;
        gtile(m, ti, cc);
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = gn * sm.Gd[(16 * ti + 4 * j + i) * LDSL + cc];
        acc = tile_mm<C / 4>(acc, 0, j, [&](int kx) { return kf(sm.Q[kx * LDK + 16 * ti + c16]); },
                             [&](int kx) { return sm.gm[kx] * sm.Ds[kx * LDSL + cc]; });
        acc = tile_mm<C / 4>(acc, 0, j, [&](int kx) { return kf(sm.K[kx * LDK + 16 * ti + c16]); },
                             [&](int kx) { return -sm.gm[kx] * sm.beta[kx] * sm.Us[kx * LDSL + cc]; });
        gnew[m] = acc;
      }
    }
    lds_barrier();
    {
      float x = 0.f;
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        if (w + BW * m >= NST) break;
        int ti, cc;
        gtile(m, ti, cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ti + 4 * j + i;
          sm.Gd[r * LDSL + cc] = gnew[m][i];
          x = fmaf(gnew[m][i], sm.Sc[r * LDSL + cc], x);
        }
      }
      cend = block_sum<E, D>(sm, x, w, l);
    }
  }
  __syncthreads();
  if (p.d_initial) {
    for (int idx = fresh(tid); idx < D * DV; idx += BT) {
      const int i = idx / DV, c = idx % DV;
      p.d_initial[sh * DD + i * D + col0 + c] = sm.Gd[i * LDSL + c];
    }
  }
}

// Adds the column slices' contributions in slice order and finishes dk,
// deta and dalpha.  One thread per 4 consecutive key channels of a
// (token, head).
__device__ inline f32x4 ld_k4(const __bf16 *k, int64_t g) {
  const bf16x4 b = *reinterpret_cast<const bf16x4 *>(k + g);
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
__device__ inline f32x4 ld_k4(const float *k, int64_t g) {
  return *reinterpret_cast<const f32x4 *>(k + g);
}

template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_finish_kernel(BwdParams p) {
  constexpr int NS = D / BwdCfg<E, D>::DV;
  const int64_t TH = p.total_tok * p.H;
  const int64_t g4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g4 >= TH * (D / 4)) return;
  const int64_t g = 4 * g4, th = g / D;
  const int i = (int)(g % D);
  f32x4 dq = zero4(), dk = zero4();
  float db = 0.f, c = 0.f;
  // the partials are read once: non-temporal loads keep them from
  // displacing the rest in the caches
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    dq += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.ws_dq + (int64_t)s * TH * D + g));
    dk += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.ws_dk + (int64_t)s * TH * D + g));
    db += p.ws_db[(int64_t)s * TH + th];
    c += p.ws_c[(int64_t)s * TH + th];
  }
  const float kk = p.ws_kk[th];
  const float eta = p.eta[th];
  const f32x4 kv = ld_k4(static_cast<const E *>(p.k), g);
  float coef;
  if (p.beta_direct) {
    coef = eta * eta;
  } else {
    const float den = kk + p.eps;
    const float beta = eta / den;
    coef = beta * beta - 2.f * beta / den;
  }
  const float f = db * coef;
  __builtin_nontemporal_store(dq, reinterpret_cast<f32x4 *>(p.dq + g));
  __builtin_nontemporal_store(
      f32x4{fmaf(f, kv[0], dk[0]), fmaf(f, kv[1], dk[1]), fmaf(f, kv[2], dk[2]), fmaf(f, kv[3], dk[3])},
      reinterpret_cast<f32x4 *>(p.dk + g));
  if (i == 0) {
    p.d_eta[th] = p.beta_direct ? db : db / (kk + p.eps);
    if (p.alpha) p.d_alpha[th] = c / p.alpha[th];
  }
}

template <typename E, int D>
hipError_t launch_bwd_t(const BwdParams &p, hipStream_t st) {
  if (p.ws_fin && p.total_tok > 0) {
    // bf16: the chunk-start states from the states-only prefill
    PrefillArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.alpha = p.alpha;
    a.eta = p.eta;
    a.cu_seqlens = p.cu_seqlens;
    a.n_seqs = p.n_seqs;
    a.seq_len_dense = p.seq_len_dense;
    a.H = p.H;
    a.D = D;
    a.eps = p.eps;
    a.beta_direct = p.beta_direct;
    a.initial_state = p.initial_state;
    a.o = p.dv;  // not written by the states-only pass
    a.final_state = p.ws_fin;
    a.ws_ckpt = p.ws_ckpt;
    hipError_t e = launch_prefill_states(a, st);
    if (e != hipSuccess) return e;
  }
  const int64_t groups = (int64_t)p.n_seqs * p.H * (D / BwdCfg<E, D>::DV);
  hipLaunchKernelGGL((bwd_kernel<E, D>), dim3((unsigned)groups), dim3(BT), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.total_tok == 0) return e;
  const int64_t n4 = p.total_tok * p.H * (D / 4);
  hipLaunchKernelGGL((bwd_finish_kernel<E, D>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams &p_in, bool bf16_inputs, hipStream_t st) {
  BwdParams p = p_in;
  if (!bf16_inputs || p.total_tok == 0) p.ws_fin = nullptr;  // fp32: the kernel's own forward sweep
  if (bf16_inputs) return p.D == 64 ? launch_bwd_t<__bf16, 64>(p, st) : launch_bwd_t<__bf16, 128>(p, st);
  return p.D == 64 ? launch_bwd_t<float, 64>(p, st) : launch_bwd_t<float, 128>(p, st);
}

}  // namespace kla
