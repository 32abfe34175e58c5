// Launch entry points of the HIP kernels, replaced for a host-only build of the
// C ABI (abk_api.cpp + pool.cpp compiled by g++ with AddressSanitizer and
// UndefinedBehaviorSanitizer). Host-only pools never launch anything, so every
// launcher reports "not supported" and no device shape is served.
#include "../../long_reasoning_kv_amd/csrc/kernels.h"

namespace abk {

hipError_t launch_append(const AppendArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode(const DecodeArgs&, int32_t, hipStream_t) { return hipErrorNotSupported; }
bool decode_stream_supported(const DevPool&, int32_t) { return false; }
int32_t decode_stream_blocks_per_cu(const DevPool&) { return 0; }
hipError_t launch_decode_stream(const StreamArgs&, int32_t, hipStream_t) { return hipErrorNotSupported; }
bool decode_mfma_supported(const DevPool&, int32_t) { return false; }
int32_t decode_mfma_waves_per_cu() { return 0; }
hipError_t launch_decode_mfma(const StreamArgs&, int32_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_free(const FreeArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prompt(const PromptArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_compress(const CompressArgs&, hipStream_t) { return hipErrorNotSupported; }
bool compress_mfma_supported(const DevPool&, int32_t) { return false; }
hipError_t launch_fill(const FillArgs&, int32_t, hipStream_t) { return hipErrorNotSupported; }
bool blockmask_supported(const DevPool&, int32_t) { return false; }
hipError_t launch_blockmask(const BlockMaskArgs&, int32_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_read(const ReadArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_export(const ExportArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(void**) { return hipErrorNotSupported; }

}  // namespace abk
