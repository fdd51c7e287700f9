// Launchers for the host-only sanitizer build of the C-ABI layer (built by
// tests/sanitize/build.py with g++ and AddressSanitizer + UBSan): every
// launch reports a HIP error, so the C-ABI's validation paths run under the
// sanitizers without a GPU or the HIP kernels.
#include "../../delta_rule_linear_amd/csrc/kla_internal.h"

namespace kla {
hipError_t launch_prefill_bf16(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_f32(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_bf16(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_f32(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_split_identity(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_split_scan(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(void **) { return hipErrorNotSupported; }
hipError_t launch_seq_order(const int32_t *, int, int32_t *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ccq_query(const CcqArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ccq_decode_step(const CcqDecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_kda(const PrefillArgs &, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_states(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd(const BwdParams &, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kla
