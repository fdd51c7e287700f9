// Curvature-conditioned read (CCQ) for the KLA path on gfx950: the query
// cleaning that runs before the prefill read, and the decode step with its
// cleaning fused in.
//
// "Don't Read Everything: A Curvature-Conditioned Query for Linear
// Attention" (sections "Derivacao Teorica" and "O Mecanismo"): the read uses
//   q_clean_t = q_t - lambda_t Sigma_t q_t,
// Sigma_t the covariance of the keys j <= t with uniform weights (the
// Hessian at q = 0 of log sum_j exp(k_j^T q)):
//   Sigma_t q = P_t q / n_t - m_t (m_t . q) / n_t^2,
//   P_t = sum_{j<=t} k_j k_j^T,  m_t = sum_{j<=t} k_j,  n_t = number of keys.
// The write is untouched, so the KLA kernels then read with q_clean.
//
// The running sums (P, m, n) are the extra state per head, one record of
// CcqStride(D) floats: [P row-major | m | n | 3 pad].
//
// Prefill pre-pass, chunk form.  For a chunk of n <= 64 tokens with sums
// (P, m, n0) at its start:
//   P_t q_t   = (Q P)_t + (lower(Q K^T) K)_t        (t >= s inside the chunk)
//   m_t       = m + prefix sums of the chunk's keys
//   m_t . q_t = m . q_t + row sums of lower(Q K^T)
//   P += K^T K (summed over the chunk first, then added: two-level sums)
// Mapping as the fp32 prefill kernel: one workgroup of 4 waves per
// (sequence, head, 64 columns), each wave owning 16 columns of P in MFMA
// accumulator tiles.  Every contraction runs on the MFMA: for bf16 inputs
// Q K^T and K^T K on the bf16 MFMA (exact products), Q P with P split into
// bf16 hi + lo, and the fp32 products (lower(Q K^T) K) on the fp32 MFMA;
// for fp32 inputs all on the fp32 MFMA.  The running key sums m_t come from
// the MFMA too (a lower ones mask per diagonal block).  The columns of
// q_clean follow the columns of P; both workgroups of a (sequence, head)
// keep the whole m.  For bf16 inputs long sequences run as two halves (a
// sums-only pass over the first halves, then both halves in parallel), so
// that two workgroups share each CU.  Output: q_clean as fp32, or as a bf16 hi / lo pair
// (q_clean = hi + lo to 2^-17) for the bf16 prefill, which reads with both
// planes in one state pass.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {
namespace {

template <typename E, int D>
struct CcqSmem {
  static constexpr int LDK = D + 4;
  static constexpr int LDP = C + 4;
  static constexpr int LDB = D + 8;  // row pitch of the bf16 keys
  // fp32 inputs: the chunk's keys and queries
  alignas(16) float Kr[sizeof(E) == 2 ? 4 : C * LDK];
  alignas(16) float Qr[sizeof(E) == 2 ? 4 : C * LDK];
  // bf16 inputs: the chunk's keys and queries as read (exact), row-major, the
  // MFMA operands (K^T K by transposing reads) and converted where an fp32
  // value is needed
  alignas(16) __bf16 Kb[sizeof(E) == 2 ? C * LDB : 8];
  alignas(16) __bf16 Qb[sizeof(E) == 2 ? C * LDB : 8];
  alignas(16) float G[C * LDP];    // lower(Q K^T), zero above the diagonal
  alignas(16) float msum[D];       // m at the chunk start (all columns)
  alignas(16) float mdp[4 * C];    // m . q_t, one partial per wave (a quarter of the columns each)
  alignas(16) float rsum[4 * C];   // row sums of lower(Q K^T), one partial per 16-column block
  alignas(16) float kp[kThreads];  // the chunk's key sums, kThreads / D partials per column
  alignas(16) float mq[C];         // m_t . q_t
  alignas(16) float lam[C];
};

// a 16-byte segment of fp32 inputs to LDS
__device__ inline void seg_to_f32(const uint4 &u, float *dst) {
  *reinterpret_cast<f32x4 *>(dst) =
      f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
}

// OUT_BF16: write q_clean as bf16 hi (qh) and lo (ql) planes; else fp32 to qh.
// SUMS_ONLY: only the running sums (the first halves of split sequences).
//
// split_mode 0: one workgroup per (sequence, head, column block) over the
// whole sequence.  Sequences of at least LMIN tokens can instead be cut at a
// chunk boundary into two halves: split_mode 1 (SUMS_ONLY) runs over the
// first halves and leaves their end sums in half_sums, at the sequence's own
// token rows (a scratch area of total_tok x H x D floats: a sequence's
// LMIN x H x D floats hold its H records); split_mode 2 then runs both
// halves, one workgroup each, the second starting from those sums, and every
// shorter sequence whole.
template <typename E, int D, bool OUT_BF16, bool SUMS_ONLY>
__global__ __launch_bounds__(kThreads) void ccq_query_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const float *__restrict__ lambda,
    const int32_t *__restrict__ cu_seqlens, int64_t seq_len_dense, int H,
    const float *__restrict__ ccq_in, float *__restrict__ ccq_out, void *__restrict__ qh,
    void *__restrict__ ql, int split_mode, float *__restrict__ half_sums) {
  using SM = CcqSmem<E, D>;
  constexpr int NB = D / DVB;
  constexpr int NST = D / 16;
  constexpr int LDK = SM::LDK, LDP = SM::LDP, LDB = SM::LDB;
  constexpr bool BF = sizeof(E) == 2;
  constexpr int SEG_EL = 16 / sizeof(E);
  constexpr int SEG_ROW = D / SEG_EL;
  constexpr int NSEG = C * SEG_ROW / kThreads;
  static_assert(NSEG * kThreads == C * SEG_ROW, "staging tiling");
  constexpr int64_t REC = (int64_t)D * D + D + 4;  // record stride (floats)
  constexpr int64_t LMIN = (REC + D - 1) / D > C + 1 ? (REC + D - 1) / D : C + 1;
  // a split sequence's H records fit its own LMIN x H x D floats of half_sums
  static_assert(REC <= LMIN * D, "the half-sums records must fit a sequence's own rows");
  static_assert(!SUMS_ONLY || BF, "the sums-only pass serves bf16 inputs");

  __shared__ SM sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int j = l >> 4, c16 = l & 15;

  const int64_t lb = logical_block();
  const int nb = (int)(lb % NB);
  const int seg = split_mode == 2 ? (int)((lb / NB) % 2) : 0;
  const int64_t sh = split_mode == 2 ? lb / (2 * NB) : lb / NB;
  const int h = (int)(sh % H);
  const int64_t s = sh / H;
  const int64_t bos = cu_seqlens ? (int64_t)cu_seqlens[s] : s * seq_len_dense;
  const int64_t eos = cu_seqlens ? (int64_t)cu_seqlens[s + 1] : bos + seq_len_dense;
  // this workgroup's tokens [lo, hi), start sums (null: zero), end sums (null: none)
  const int64_t len = eos - bos;
  const bool split = split_mode != 0 && len >= LMIN;
  const int64_t mid = bos + (int64_t)C * (((len + C - 1) / C + 1) / 2);
  float *const hrec = split ? half_sums + bos * H * (int64_t)D + (int64_t)h * REC : nullptr;
  int64_t lo = bos, hi = eos;
  const float *rin = ccq_in ? ccq_in + sh * REC : nullptr;
  float *rout = ccq_out ? ccq_out + sh * REC : nullptr;
  if (split_mode == 1) {
    if (!split) return;
    hi = mid;
    rout = hrec;
  } else if (split_mode == 2) {
    if (seg == 1) {
      if (!split) return;
      lo = mid;
      rin = hrec;
    } else if (split) {
      hi = mid;
      rout = nullptr;
    }
  }
  const int cl = 16 * w + c16;       // column within this workgroup's block
  const int col = nb * DVB + cl;     // column of P and of q_clean

  // G above the diagonal blocks stays zero, and so do the row-sum partials
  // of the blocks above the diagonal (never written)
  for (int i = tid; i < C * LDP; i += kThreads) sm.G[i] = 0.f;
  for (int i = tid; i < 4 * C; i += kThreads) sm.rsum[i] = 0.f;

  // start sums: P tiles (rows 16t+4j+i, column col), m, n
  f32x4 P[NST];
  float n0;
  {
    const rsrc_t rr = make_rsrc(rin ? rin : lambda, rin ? REC * 4 : 0);
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) P[t][i] = buf_ld4(rr, (uint32_t)(((16 * t + 4 * j + i) * D + col) * 4));
    if (tid < D) sm.msum[tid] = buf_ld4(rr, (uint32_t)((D * D + tid) * 4));
    n0 = buf_ld4(rr, (uint32_t)((D * D + D) * 4));
  }

  uint4 kreg[NSEG], qreg[NSEG];
  float lreg = 0.f;
  auto fetch = [&](int64_t t0) {
    const int64_t nn = (hi - t0) < C ? (hi - t0) : C;
    const int64_t rowb = (int64_t)H * D * sizeof(E);
    const rsrc_t rk = make_rsrc(k + t0 * H * (int64_t)D, nn * rowb);
    const rsrc_t rq = make_rsrc(q + t0 * H * (int64_t)D, nn * rowb);
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      const uint32_t off = (uint32_t)((r * H + h) * D + cs * SEG_EL) * sizeof(E);
      kreg[u] = buf_ld16(rk, off);
      if constexpr (!SUMS_ONLY) qreg[u] = buf_ld16(rq, off);
    }
    if (!SUMS_ONLY && w == 0) {
      const rsrc_t rl = make_rsrc(lambda + t0 * H, nn * H * 4);
      lreg = buf_ld4(rl, (uint32_t)(l * H + h) * 4);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int sg = u * kThreads + tid, r = sg / SEG_ROW, cs = sg % SEG_ROW;
      if constexpr (BF) {
        *reinterpret_cast<uint4 *>(&sm.Kb[r * LDB + cs * SEG_EL]) = kreg[u];
        if constexpr (!SUMS_ONLY) *reinterpret_cast<uint4 *>(&sm.Qb[r * LDB + cs * SEG_EL]) = qreg[u];
      } else {
        seg_to_f32(kreg[u], &sm.Kr[r * LDK + cs * SEG_EL]);
        seg_to_f32(qreg[u], &sm.Qr[r * LDK + cs * SEG_EL]);
      }
    }
    if (!SUMS_ONLY && w == 0) sm.lam[l] = lreg;
  };
  // element (token r, feature c) of the chunk's keys / queries as fp32
  auto kval = [&](int r, int c) __attribute__((always_inline)) -> float {
    if constexpr (BF) return static_cast<float>(sm.Kb[r * LDB + c]);
    else return sm.Kr[r * LDK + c];
  };
  auto qval = [&](int r, int c) __attribute__((always_inline)) -> float {
    if constexpr (BF) return static_cast<float>(sm.Qb[r * LDB + c]);
    else return sm.Qr[r * LDK + c];
  };

  fetch(lo);
  stage();
  for (int64_t tok0 = lo; tok0 < hi; tok0 += C) {
    const int n = (int)((hi - tok0) < C ? (hi - tok0) : C);
    lds_barrier();  // chunk staged (and m of the chunk start final)
    fetch(tok0 + C);

    f32x4 PQ[4];  // (Q P + lower(Q K^T) K)[16bi + 4j + i][col]
    if constexpr (!SUMS_ONLY) {
    // ---- lower(Q K^T) tiles, Q P for this wave's columns, m . q_t ----------
    {
      // tiles (bi, bj), bj <= bi, numbered 0..9 in row order; wave w takes
      // tiles w, w + 4, w + 8
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int tn = w + 4 * u;
        if (tn < 10) {
          const int bi = (tn >= 1) + (tn >= 3) + (tn >= 6);
          const int bj = tn - bi * (bi + 1) / 2;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if constexpr (BF) {
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb)
              acc = mma(*reinterpret_cast<const bf16x8 *>(&sm.Qb[(16 * bi + c16) * LDB + 32 * kb + 8 * j]),
                        *reinterpret_cast<const bf16x8 *>(&sm.Kb[(16 * bj + c16) * LDB + 32 * kb + 8 * j]), acc);
          } else {
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += 4)
              acc = mma(sm.Qr[(16 * bi + c16) * LDK + k0 + j], sm.Kr[(16 * bj + c16) * LDK + k0 + j], acc);
          }
          // acc[i] = (Q K^T)[16bi + 4j + i][16bj + c16]; its row sums over
          // the tile's 16 columns (the 16 lanes of group j, one DPP row) go to
          // rsum[bj]
          float rs[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int R = 16 * bi + 4 * j + i, Sc = 16 * bj + c16;
            const float g = R >= Sc ? acc[i] : 0.f;
            sm.G[R * LDP + Sc] = g;
            rs[i] = g;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) rs[i] = group_sum<16>(rs[i]);  // DPP within the 16-lane row
          if (c16 < 4)
            sm.rsum[bj * C + 16 * bi + 4 * j + c16] = c16 == 0 ? rs[0] : c16 == 1 ? rs[1] : c16 == 2 ? rs[2] : rs[3];
        }
      }
    }
    if constexpr (BF) {
      // P split into bf16 hi + lo (to 2^-17) and used in place as the B
      // operand of the 32-deep bf16 MFMA (tiles 2kk, 2kk+1 joined: lane group
      // j holds rows 32kk + 4j + i and 32kk + 16 + 4j + i); the A operand
      // reads the query columns in the same order.  Hi and lo products go to
      // separate MFMAs.
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) PQ[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NST / 2; ++kk) {
        const Split8 pf = join(split4(P[2 * kk]), split4(P[2 * kk + 1]));
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          const __bf16 *row = &sm.Qb[(16 * bi + c16) * LDB + 32 * kk];
          const bf16x8 a = __builtin_shufflevector(*reinterpret_cast<const bf16x4 *>(row + 4 * j),
                                                   *reinterpret_cast<const bf16x4 *>(row + 16 + 4 * j),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
          PQ[bi] = mma(a, pf.hi, PQ[bi]);
          PQ[bi] = mma(a, pf.lo, PQ[bi]);
        }
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc = mma(sm.Qr[(16 * bi + c16) * LDK + 16 * t + 4 * j + i], P[t][i], acc);
        PQ[bi] = acc;  // (Q P)[16bi + 4j + i][col]
      }
    }
    {
      // m . q_t over this wave's quarter of the columns (token l)
      constexpr int QW = D / 4;
      const float *mrow = &sm.msum[QW * w];
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < QW; c += 4) {
        f32x4 x;
        if constexpr (BF) {
          const bf16x4 b = *reinterpret_cast<const bf16x4 *>(&sm.Qb[l * LDB + QW * w + c]);
          x = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
        } else {
          x = *reinterpret_cast<const f32x4 *>(&sm.Qr[l * LDK + QW * w + c]);
        }
        const f32x4 m = *reinterpret_cast<const f32x4 *>(mrow + c);
        d += x[0] * m[0] + x[1] * m[1] + x[2] * m[2] + x[3] * m[3];
      }
      sm.mdp[w * C + l] = d;
    }
    }  // !SUMS_ONLY
    lds_barrier();

    // ---- m_t . q_t = m . q_t + row sums of lower(Q K^T) -----------------------
    if (!SUMS_ONLY && w == 0) {
      float rs = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) rs += sm.mdp[u * C + l] + sm.rsum[u * C + l];
      sm.mq[l] = rs;
    }
    lds_barrier();

    // ---- P_t q_t = (Q P)_t + (lower(Q K^T) K)_t; q_clean -----------------------
    f32x4 Kc[4];  // K[16mt + 4j + i][col], the B operand of the two products below
    if constexpr (!SUMS_ONLY) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Kc[mt][i] = kval(16 * mt + 4 * j + i, col);
    // m_t for this lane's column: the chunk-start m plus running key sums, on
    // the MFMA with a lower ones mask per diagonal block and the block
    // totals (row 15 of each block, held by lane group 3) carried
    f32x4 cmv[4];
    {
      float carry = sm.msum[col];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) a = mma(c16 >= 4 * j + i ? 1.f : 0.f, Kc[bi][i], a);
#pragma unroll
        for (int i = 0; i < 4; ++i) cmv[bi][i] = carry + a[i];
        carry += __shfl(a[3], 48 + c16, 64);
      }
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      f32x4 acc = PQ[bi];
#pragma unroll
      for (int mt = 0; mt <= bi; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mma(sm.G[(16 * bi + c16) * LDP + 16 * mt + 4 * j + i], Kc[mt][i], acc);
      PQ[bi] = acc;
    }
    {
      // range-checked stores: rows past the chunk's n tokens are dropped
      constexpr int OSZ = OUT_BF16 ? 2 : 4;
      const int64_t base = tok0 * H * (int64_t)D, bytes = (int64_t)n * H * D * OSZ;
      const rsrc_t rh = make_rsrc(static_cast<char *>(qh) + base * OSZ, bytes);
      const rsrc_t rl = make_rsrc(OUT_BF16 ? static_cast<char *>(ql) + base * OSZ : static_cast<char *>(qh), bytes);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * bi + 4 * j + i;
          const float inv = 1.f / (n0 + (float)(r + 1));
          const float sq = PQ[bi][i] * inv - (cmv[bi][i] * inv) * (sm.mq[r] * inv);
          const float qc = qval(r, col) - sm.lam[r] * sq;
          const uint32_t off = (uint32_t)(((r * H + h) * D + col) * OSZ);
          if constexpr (OUT_BF16) {
            const __bf16 hi = static_cast<__bf16>(qc);
            const __bf16 lo = static_cast<__bf16>(qc - static_cast<float>(hi));
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, hi), rh, (int)off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, lo), rl, (int)off, 0, 0);
          } else {
            buf_st4(rh, off, qc);
          }
        }
    }

    }  // !SUMS_ONLY
    // ---- P += K^T K (the chunk's sum first), m, n -----------------------------
    {
      f32x4 Pc[NST];
      // bf16: (K^T K)[16t + 4j + i][col] with A = K^T rows 16t + c16 and B = K^T
      // row col, both by transposing reads of the row-major keys; lane group j
      // takes tokens 32kb + 4j .. +3 and 32kb + 16 + 4j .. +3 in both operands
      // (the same order of the contraction index on both sides)
      [[maybe_unused]] bf16x8 bk[C / 32];
      if constexpr (BF) {
        const __bf16 *pb = &sm.Kb[nb * DVB + 16 * w + 4 * (c16 & 3)];
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb)
          bk[kb] = __builtin_shufflevector(ld_tr(pb + (32 * kb + 4 * j + (c16 >> 2)) * LDB),
                                           ld_tr(pb + (32 * kb + 16 + 4 * j + (c16 >> 2)) * LDB),
                                           0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int t = 0; t < NST; ++t) {
        Pc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
          const __bf16 *pa = &sm.Kb[16 * t + 4 * (c16 & 3)];
#pragma unroll
          for (int kb = 0; kb < C / 32; ++kb) {
            const bf16x8 a = __builtin_shufflevector(ld_tr(pa + (32 * kb + 4 * j + (c16 >> 2)) * LDB),
                                                     ld_tr(pa + (32 * kb + 16 + 4 * j + (c16 >> 2)) * LDB),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
            Pc[t] = mma(a, bk[kb], Pc[t]);
          }
        } else {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              Pc[t] = mma(sm.Kr[(16 * mt + 4 * j + i) * LDK + 16 * t + c16], Kc[mt][i], Pc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < NST; ++t) P[t] += Pc[t];
    }
    {
      // the chunk's key sums: thread tid sums a 1 / (kThreads / D) share of
      // the tokens for column tid % D
      constexpr int TP = C * D / kThreads;
      const int c = tid % D, part = tid / D;
      float a = 0.f;
#pragma unroll 8
      for (int t = 0; t < TP; ++t) a += kval(part * TP + t, c);
      sm.kp[tid] = a;
    }
    lds_barrier();  // every read of this chunk's K, Q, m is done
    if (tid < D) {
      float a = 0.f;
#pragma unroll
      for (int u = 0; u < kThreads / D; ++u) a += sm.kp[u * D + tid];
      sm.msum[tid] += a;
    }
    n0 += (float)n;
    stage();  // writes K, Q, lambda only: no reader of them is left in this chunk
  }

  if (rout) {
    float *rec = rout;
#pragma unroll
    for (int t = 0; t < NST; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[(16 * t + 4 * j + i) * D + col] = P[t][i];
    if (nb == 0) {
      if (tid < D) rec[D * D + tid] = sm.msum[tid];
      if (tid < 4) rec[D * D + D + tid] = tid == 0 ? n0 : 0.f;  // n, then the zero pad
    }
  }
}

// One decode token, fused: the sums take the new key, q_clean is formed, and
// the KLA decode step reads with it (x = S^T k, y = S^T q_clean from one read
// of S; e = v - alpha x; o = alpha y + beta (k . q_clean) e; S <- alpha S +
// beta k e^T).  One workgroup of 512 threads per (sequence, head); thread
// (row group, column group) holds rows rg + NRG i, columns 4 cq .. 4 cq + 3 of
// both P and S, loaded together at the start.  Both go back with
// non-temporal stores (read again only by the next step).  q_clean is also
// written to qc_out.
constexpr int kDecThreads = 512;
template <typename E, int D>
__global__ __launch_bounds__(kDecThreads) void ccq_decode_step_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ lambda, const float *__restrict__ alpha, const float *__restrict__ eta,
    float *__restrict__ ccq_state, float *__restrict__ state, float *__restrict__ o,
    float *__restrict__ qc_out, float eps, int beta_direct) {
  constexpr int NQ = D / 4, NRG = kDecThreads / NQ, RPT = D / NRG;
  static_assert(NQ * NRG == kDecThreads && RPT * NRG == D, "tiling");
  constexpr int64_t REC = (int64_t)D * D + D + 4;
  __shared__ float sq[D], sk[D], sv[D], sqc[D], se[D], sm_m[D], red[2];
  __shared__ float px[NRG][D], py[NRG][D];
  const int64_t sh = blockIdx.x;
  const int t = threadIdx.x, cq = t % NQ, rg = t / NQ;
  float *rec = ccq_state + sh * REC;
  float *Sg = state + sh * (int64_t)(D * D);
  float4 p[RPT], s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) p[i] = *reinterpret_cast<const float4 *>(rec + (rg + NRG * i) * D + 4 * cq);
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = *reinterpret_cast<const float4 *>(Sg + (rg + NRG * i) * D + 4 * cq);
  if (t < D) {
    sq[t] = static_cast<float>(q[sh * D + t]);
    sk[t] = static_cast<float>(k[sh * D + t]);
    sv[t] = static_cast<float>(v[sh * D + t]);
  }
  const float a = alpha ? alpha[sh] : 1.f;
  const float et = eta[sh];
  __syncthreads();

  // ---- sums: P += k k^T, m += k, n += 1; then q_clean -------------------------
  // partial (P q) over this thread's rows for its 4 columns (P is symmetric:
  // (P q)_c = sum_r P[r][c] q[r])
  {
    const float4 kc = *reinterpret_cast<const float4 *>(&sk[4 * cq]);
    float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + NRG * i;
      const float kr = sk[r], qr = sq[r];
      p[i].x += kr * kc.x; p[i].y += kr * kc.y; p[i].z += kr * kc.z; p[i].w += kr * kc.w;
      acc.x += p[i].x * qr; acc.y += p[i].y * qr; acc.z += p[i].z * qr; acc.w += p[i].w * qr;
      __builtin_nontemporal_store(f32x4{p[i].x, p[i].y, p[i].z, p[i].w},
                                  reinterpret_cast<f32x4 *>(rec + r * D + 4 * cq));
    }
    *reinterpret_cast<float4 *>(&px[rg][4 * cq]) = acc;
  }
  if (t < 64) {
    // m += k, n += 1 and m . q (wave 0)
    float mq = 0.f;
    for (int c = t; c < D; c += 64) {
      const float m = rec[D * D + c] + sk[c];
      rec[D * D + c] = m;
      sm_m[c] = m;
      mq += m * sq[c];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mq += __shfl_xor(mq, off, 64);
    if (t == 0) {
      const float n = rec[D * D + D] + 1.f;
      rec[D * D + D] = n;
      red[0] = mq;
      red[1] = n;
    }
  }
  __syncthreads();
  if (t < D) {
    float pq = 0.f;
#pragma unroll
    for (int r = 0; r < NRG; ++r) pq += px[r][t];
    const float inv = 1.f / red[1];
    const float m = sm_m[t];
    const float sg = pq * inv - (m * inv) * (red[0] * inv);
    const float qc = sq[t] - lambda[sh] * sg;
    sqc[t] = qc;
    qc_out[sh * D + t] = qc;
  }
  __syncthreads();  // q_clean complete; every read of px done

  // ---- KLA decode step with q_clean ------------------------------------------
  // k.k and k.q_clean: every wave reduces its own copy (fixed order)
  float kk = 0.f, kq = 0.f;
  {
    const int l = t & 63;
#pragma unroll
    for (int i = l; i < D; i += 64) {
      kk += sk[i] * sk[i];
      kq += sk[i] * sqc[i];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      kk += __shfl_xor(kk, off, 64);
      kq += __shfl_xor(kq, off, 64);
    }
  }
  const float beta = beta_direct ? et : et / (kk + eps);
  {
    float4 xs = {0.f, 0.f, 0.f, 0.f}, ys = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float kr = sk[rg + NRG * i], qr = sqc[rg + NRG * i];
      xs.x += s[i].x * kr; xs.y += s[i].y * kr; xs.z += s[i].z * kr; xs.w += s[i].w * kr;
      ys.x += s[i].x * qr; ys.y += s[i].y * qr; ys.z += s[i].z * qr; ys.w += s[i].w * qr;
    }
    *reinterpret_cast<float4 *>(&px[rg][4 * cq]) = xs;
    *reinterpret_cast<float4 *>(&py[rg][4 * cq]) = ys;
  }
  __syncthreads();
  if (t < D) {
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
      x += px[r][t];
      y += py[r][t];
    }
    const float e = sv[t] - a * x;
    se[t] = e;
    o[sh * D + t] = a * y + beta * kq * e;
  }
  __syncthreads();
  const float4 e4 = *reinterpret_cast<const float4 *>(&se[4 * cq]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float bk = beta * sk[rg + NRG * i];
    const f32x4 r = {a * s[i].x + bk * e4.x, a * s[i].y + bk * e4.y, a * s[i].z + bk * e4.z,
                     a * s[i].w + bk * e4.w};
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4 *>(Sg + (rg + NRG * i) * D + 4 * cq));
  }
}

}  // namespace

hipError_t launch_ccq_query(const CcqArgs &a, hipStream_t st) {
  const int64_t grid = (int64_t)a.n_seqs * a.H * (a.D / DVB);
  const dim3 b(kThreads);
#define KLA_CCQ_LAUNCH(E, DD, BF, SO, MODE, G)                                                     \
  hipLaunchKernelGGL((ccq_query_kernel<E, DD, BF, SO>), dim3((unsigned)(G)), b, 0, st,             \
                     static_cast<const E *>(a.q), static_cast<const E *>(a.k), a.lambda,          \
                     a.cu_seqlens, a.seq_len_dense, a.H, a.ccq_in, a.ccq_out, a.qh, a.ql, MODE,   \
                     a.half_sums)
  if (a.bf16_inputs && a.half_sums) {
    // long sequences in two halves: the first halves' sums, then both halves
    if (a.D == 128) {
      KLA_CCQ_LAUNCH(__bf16, 128, true, true, 1, grid);
      KLA_CCQ_LAUNCH(__bf16, 128, true, false, 2, 2 * grid);
    } else {
      KLA_CCQ_LAUNCH(__bf16, 64, true, true, 1, grid);
      KLA_CCQ_LAUNCH(__bf16, 64, true, false, 2, 2 * grid);
    }
  } else if (a.bf16_inputs) {
    if (a.D == 128) KLA_CCQ_LAUNCH(__bf16, 128, true, false, 0, grid); else KLA_CCQ_LAUNCH(__bf16, 64, true, false, 0, grid);
  } else {
    if (a.D == 128) KLA_CCQ_LAUNCH(float, 128, false, false, 0, grid); else KLA_CCQ_LAUNCH(float, 64, false, false, 0, grid);
  }
#undef KLA_CCQ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_ccq_decode_step(const CcqDecodeArgs &a, hipStream_t st) {
  const dim3 g((unsigned)((int64_t)a.n_seqs * a.H)), b(kDecThreads);
#define KLA_CCQ_DEC_LAUNCH(E, DD)                                                                   \
  hipLaunchKernelGGL((ccq_decode_step_kernel<E, DD>), g, b, 0, st, static_cast<const E *>(a.q),     \
                     static_cast<const E *>(a.k), static_cast<const E *>(a.v), a.lambda, a.alpha,    \
                     a.eta, a.ccq_state, a.state, a.o, a.q_clean, a.eps, a.beta_direct)
  if (a.bf16_inputs) {
    if (a.D == 128) KLA_CCQ_DEC_LAUNCH(__bf16, 128); else KLA_CCQ_DEC_LAUNCH(__bf16, 64);
  } else {
    if (a.D == 128) KLA_CCQ_DEC_LAUNCH(float, 128); else KLA_CCQ_DEC_LAUNCH(float, 64);
  }
#undef KLA_CCQ_DEC_LAUNCH
  return hipGetLastError();
}

}  // namespace kla
