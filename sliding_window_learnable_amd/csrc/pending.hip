// Launchers not implemented yet: they report an error and launch nothing.
#include "launch.h"
namespace swa {
hipError_t launch_stream_bf16(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
}
