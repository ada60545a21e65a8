// Sol-Attn2 kernels (placeholder launchers until the FP8 path is written).
#include "common.h"
#include "kernels.h"
namespace solattn {
hipError_t launch_quant_summary(const uint16_t*, const uint16_t*, const uint16_t*, Shape, const Workspace&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_qhat(Shape, const Workspace&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_groups(const uint16_t*, Shape, const Workspace&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fused2(const uint16_t*, uint16_t*, Shape, const Workspace&, int, int, uint64_t*, hipStream_t) { return hipErrorNotSupported; }
}
