// prefill.hip -- gfx950 chunked-prefill kernel of libpa (matrix-core path).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

int launch_prefill(const DecodeLaunch &l, void *stream) {
    (void)l;
    (void)stream;
    return (int)hipErrorNotSupported;
}

}  // namespace pa
