// Streaming-layout instances of the persistent kernel.
#include "pk_persistent.h"

using namespace pkd;

const void* pkk_stream_fn(int dtype, bool has_b) {
    if (dtype == PK_F64)
        return has_b ? reinterpret_cast<const void*>(&pk_persistent<double, true, PK_LAYOUT_STREAM, 0, false>)
                     : reinterpret_cast<const void*>(&pk_persistent<double, false, PK_LAYOUT_STREAM, 0, false>);
    return has_b ? reinterpret_cast<const void*>(&pk_persistent<float, true, PK_LAYOUT_STREAM, 0, false>)
                 : reinterpret_cast<const void*>(&pk_persistent<float, false, PK_LAYOUT_STREAM, 0, false>);
}
