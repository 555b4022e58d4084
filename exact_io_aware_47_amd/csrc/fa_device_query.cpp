// fa_device_query.cpp -- properties of the current HIP device that size launches.
#include "fa_kernels.h"

namespace fa {

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    return n;
  // No usable device (or a failed query): clear the error so that the next
  // launch check does not report it, and size for the whole chip.
  (void)hipGetLastError();
  return kFullChipCUs;
}

}  // namespace fa
