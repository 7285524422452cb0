// placeholder until the matrix-core linear-attention path lands
#include "kernels.hpp"
namespace la {
bool la_mfma_supported(int, int, int, int) { return false; }
size_t la_mfma_workspace_bytes(int, int, int, int, int, int) { return 0; }
hipError_t launch_la_mfma(int, int, int, const void*, const void*, const void*, const float*,
                          const float*, void*, float*, float*, void*, hipStream_t) {
    return hipErrorInvalidValue;
}
}  // namespace la
