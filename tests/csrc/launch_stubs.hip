// launch_stubs.hip -- stand-ins for the launchers of the two kernel translation units
// (the recurrent and the chunked kernels) in the sanitized host build of the library's
// argument checks, which leaves those units out to keep the build to seconds.  The checks
// under test refuse their arguments before any launch, so reaching a stand-in is a test
// failure: it reports and aborts.
#include <stdio.h>
#include <stdlib.h>

#include "kda_internal.h"

namespace kda {

static hipError_t reached(const char *what) {
    fprintf(stderr, "launch stand-in reached: %s\n", what);
    abort();
    return hipErrorInvalidValue;
}

hipError_t launch_recurrent(const LayerParams &, int, int, hipStream_t) { return reached("launch_recurrent"); }
hipError_t launch_chunked_throughput(const LayerParams &, int, hipStream_t) {
    return reached("launch_chunked_throughput");
}
hipError_t launch_chunked_segments(const LayerParams &, int, int, hipStream_t) {
    return reached("launch_chunked_segments");
}

}  // namespace kda
