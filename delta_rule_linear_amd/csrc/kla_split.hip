// Split-sequence prefill: the scan between the two passes of the prefill
// kernel (modes 1 and 2 of resolve_work in kla_prefill.hip).
//
// Each chunk of the recurrence, and so each segment of chunks, maps the
// state affinely: S_end = A S_start + B, with A depending on the keys and
// gates only and B the end state from a zero start.  This is the chunk form
// the KLA technical summary keeps from Gated DeltaNet ("Resumo Tecnico:
// Atencao Linear Kaczmarz (KLA)", section "Implementacao"): the state update
// of a chunk is linear in the chunk-start state.  Maps compose, so after
// pass 1 has produced (A_p, B_p) for segments p = 0..P-2, the start state
// of every segment follows by a sequential scan over P-1 small products:
//   S_0 = initial state (or 0),  S_{p+1} = A_p S_p + B_p.
// Pass 2 then runs all segments at once from those starts.
//
// The no-allocation variant of the split-sequence prefill keeps the maps and
// start states in `scratch`, a file-scope device array below, instead of a
// caller workspace.  Host code never passes the array's name to a kernel
// (in host code it is a stand-in, not a device address): the device address
// is taken with hipGetSymbolAddress, once per device with that device
// current, and kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kla.h"
#include "kla_internal.h"

// Scratch of kla_fwd_chunked_split_noalloc; every GPU the library runs on
// holds one copy until the process ends.  Calls on one GPU share it.
static __device__ __align__(256) float scratch[KLA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace kla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kScanThreads = 256;
constexpr int kCols = 16;  // state columns per scan workgroup

// ws_a[m] <- I (D x D) for every m < count.
template <int D>
__global__ __launch_bounds__(256) void identity_kernel(float *__restrict__ ws_a, int64_t count) {
  const int64_t total4 = count * D * D / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = 4 * i;
    const int r = (int)((e / D) % D), c = (int)(e % D);  // four consecutive columns of row r
    float4 x;
    x.x = (c == r) ? 1.f : 0.f;
    x.y = (c + 1 == r) ? 1.f : 0.f;
    x.z = (c + 2 == r) ? 1.f : 0.f;
    x.w = (c + 3 == r) ? 1.f : 0.f;
    reinterpret_cast<float4 *>(ws_a)[i] = x;
  }
}

// One workgroup of four waves per (sequence, head, block of 16 state
// columns).  The running start state (D x 16) and the current A_p (D x D)
// live in LDS; each step S_{p+1} = A_p S_p + B_p runs on the fp32 MFMA
// (v_mfma_f32_16x16x4_f32), wave w taking row blocks w, w + 4 (D = 128) of
// the 16-column block, its accumulators started from B_p.
template <int D>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const float *__restrict__ S0,
                                                             const float *__restrict__ ws_a,
                                                             const float *__restrict__ ws_b,
                                                             float *__restrict__ ws_s, int H,
                                                             int P) {
  constexpr int NCB = D / kCols;
  constexpr int LDA = D + 4;          // A rows: lanes of a 16 x 4 operand read hit distinct banks
  constexpr int NRT = D / 64;         // row blocks per wave
  __shared__ float As[D * LDA];
  __shared__ float Ss[D * kCols];
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, j = l >> 4, c16 = l & 15;
  const int cb = (int)(blockIdx.x % NCB);
  const int64_t sh = blockIdx.x / NCB;
  constexpr int64_t DD = (int64_t)D * D;
  const int col0 = cb * kCols;

  // S_0: the caller's start state or zero, also copied to ws_s[.., 0] so
  // pass 2 never reads the caller's buffer (which may be the final state).
  for (int i = tid; i < D * kCols; i += kScanThreads) {
    const int rr = i / kCols, cc = i % kCols;
    const float x = S0 ? S0[sh * DD + (int64_t)rr * D + col0 + cc] : 0.f;
    Ss[i] = x;
    ws_s[(sh * P) * DD + (int64_t)rr * D + col0 + cc] = x;
  }
  for (int p = 0; p + 1 < P; ++p) {
    const float *A = ws_a + (sh * (P - 1) + p) * DD;
    const float *B = ws_b + (sh * (P - 1) + p) * DD;
    for (int i = tid; i < D * D / 4; i += kScanThreads) {
      const int rr = (4 * i) / D, cc = (4 * i) % D;
      *reinterpret_cast<float4 *>(&As[rr * LDA + cc]) = reinterpret_cast<const float4 *>(A)[i];
    }
    f32x4 acc[NRT];
#pragma unroll
    for (int m = 0; m < NRT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] = B[(int64_t)(16 * (w + 4 * m) + 4 * j + i) * D + col0 + c16];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NRT; ++m) {
      const int r0 = 16 * (w + 4 * m);
#pragma unroll 8
      for (int st = 0; st < D / 4; ++st) {
        const int kx = 4 * st + j;
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(As[(r0 + c16) * LDA + kx], Ss[kx * kCols + c16], acc[m],
                                                       0, 0, 0);
      }
    }
    __syncthreads();  // every wave has read Ss and As
    float *dst = ws_s + (sh * P + p + 1) * DD + col0 + c16;
#pragma unroll
    for (int m = 0; m < NRT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * (w + 4 * m) + 4 * j + i;
        Ss[rr * kCols + c16] = acc[m][i];
        dst[(int64_t)rr * D] = acc[m][i];
      }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_split_identity(const PrefillArgs &a, hipStream_t st) {
  const int64_t count = (int64_t)a.n_seqs * a.H * (a.n_splits - 1);
  const int64_t total4 = count * a.D * a.D / 4;
  const int64_t blocks = (total4 + 255) / 256 < 4096 ? (total4 + 255) / 256 : 4096;
  if (a.D == 128)
    hipLaunchKernelGGL((identity_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, st, a.ws_a,
                       count);
  else
    hipLaunchKernelGGL((identity_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, st, a.ws_a,
                       count);
  return hipGetLastError();
}

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_split_scan(const PrefillArgs &a, hipStream_t st) {
  const int64_t grid = (int64_t)a.n_seqs * a.H * (a.D / kCols);
  if (a.D == 128)
    hipLaunchKernelGGL((scan_kernel<128>), dim3((unsigned)grid), dim3(kScanThreads), 0, st,
                       a.initial_state, a.ws_a, a.ws_b, const_cast<float *>(a.ws_s), a.H,
                       a.n_splits);
  else
    hipLaunchKernelGGL((scan_kernel<64>), dim3((unsigned)grid), dim3(kScanThreads), 0, st,
                       a.initial_state, a.ws_a, a.ws_b, const_cast<float *>(a.ws_s), a.H,
                       a.n_splits);
  return hipGetLastError();
}

}  // namespace kla
