// Streaming-layout instances of the persistent kernel for float.
#include "pk_persistent.h"

using namespace pkd;

const void* pkk_stream_fn_f32(bool has_b) {
    return has_b ? reinterpret_cast<const void*>(&pk_persistent<float, true, PK_LAYOUT_STREAM, 0, false>)
                 : reinterpret_cast<const void*>(&pk_persistent<float, false, PK_LAYOUT_STREAM, 0, false>);
}
