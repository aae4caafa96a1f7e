// placeholder until the matrix-core kernel lands
#include "lla_internal.h"
#include "../../include/lla.h"
namespace lla {
size_t mfma_workspace_bytes(int, int, int) { return 0; }
bool mfma_supported(int, int) { return false; }
hipError_t launch_mfma(const FwdParams&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace lla
