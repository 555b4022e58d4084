#include "fa_device.hpp"
#include "fa_kernels.h"
namespace fa {
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}
