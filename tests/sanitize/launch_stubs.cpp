// Stand-ins for the device launchers (a8r_kernels.hip), for the CPU sanitizer
// build of the host side (a8r_host.cpp) in tests/test_host_sanitized.py.  That
// build exercises the ledger, argument validation and layout code under
// AddressSanitizer and UndefinedBehaviorSanitizer without a GPU: no path it
// runs reaches a launcher, and if one did the call would fail with
// hipErrorNoDevice, which the host code reports as A8R_EDEVICE.
#include "a8r_internal.h"

namespace a8r {

hipError_t launch_reset(const Geometry&, const StreamBatch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rebase(const Geometry&, int, const StreamBatch&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append_prefix(const Geometry&, int, const StreamBatch&, int, const void*, const void*,
                                hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_export_prefix(const Geometry&, int, const StreamBatch&, int, void*, void*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_append(const Geometry&, int, const StreamBatch&, int, const void*, const void*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_attention(const Geometry&, int, const StreamBatch&, int, const void*, void*, bool, int,
                            hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t static_scratch(int, void**) { return hipErrorNoDevice; }
hipError_t launch_rebuild(const Geometry&, int, const StreamBatch&, int, int, const void*, const void*, const void*,
                          hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_append_decode(const Geometry&, int, const StreamBatch&, const void*, const void*, const void*,
                                void*, bool, int, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_append_chunk(const Geometry&, int, const StreamBatch&, int, const void*, const void*,
                               const void*, void*, bool, int, hipStream_t) {
    return hipErrorNoDevice;
}

}  // namespace a8r
