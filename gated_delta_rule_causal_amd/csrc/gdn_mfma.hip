// placeholder until the matrix-core gated-delta path lands
#include "kernels.hpp"
namespace la {
bool gdn_mfma_supported(int, int, int, int) { return false; }
size_t gdn_mfma_workspace_bytes(int, int, int, int, int, int) { return 0; }
hipError_t launch_gdn_mfma(int, int, int, const void*, const void*, const void*, const float*,
                           const float*, const float*, void*, float*, void*, hipStream_t) {
    return hipErrorInvalidValue;
}
}  // namespace la
