// fa_launch_stubs.cpp -- host-only stand-ins for the kernel launchers, so that
// the C ABI layer (fa_api.cpp) can be built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer and driven by the CPU ABI tests without a
// GPU.  Every launcher only counts its calls; nothing touches device memory.
#include <atomic>

#include "fa_kernels.h"

namespace {
std::atomic<int> g_launches{0};
}

namespace fa {

int device_cu_count() { return kFullChipCUs; }

hipError_t launch_fwd(const FwdArgs&, hipStream_t) { g_launches++; return hipSuccess; }
hipError_t launch_fwd_fp8(const Fp8FwdArgs&, hipStream_t) { g_launches++; return hipSuccess; }
hipError_t launch_bwd(const BwdArgs&, int, hipStream_t) { g_launches++; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { g_launches++; return hipSuccess; }

// A fake, never dereferenced address for the allocation-free decode's scratch.
hipError_t decode_scratch_area(void** out) { *out = (void*)0x20000; return hipSuccess; }

// The FP8 forward's staging area: V transposed in 64-key tiles of one byte
// per element (the layout the staging kernel writes).
size_t fp8_vt_bytes(int B, int Hkv, int Nk, int d) { return (size_t)B * Hkv * ((Nk + 63) / 64) * 64 * d; }

}  // namespace fa

// Number of launcher calls so far (the tests read it through ctypes).
extern "C" int fa_stub_launch_count() { return g_launches.load(); }
