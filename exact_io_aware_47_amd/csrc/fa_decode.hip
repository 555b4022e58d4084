#include "fa_device.hpp"
#include "fa_kernels.h"
namespace fa {
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
}
