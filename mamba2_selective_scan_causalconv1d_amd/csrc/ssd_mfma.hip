// Chunked selective scan on MFMA (bf16, P = 64, N = 128) -- not yet enabled.
#include "common.h"

namespace m2 {
hipError_t launch_scan_mfma(const ScanArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace m2
