// Streaming-layout instances of the persistent kernel for double.
#include "pk_persistent.h"

using namespace pkd;

const void* pkk_stream_fn_f64(bool has_b) {
    return has_b ? reinterpret_cast<const void*>(&pk_persistent<double, true, PK_LAYOUT_STREAM, 0, false>)
                 : reinterpret_cast<const void*>(&pk_persistent<double, false, PK_LAYOUT_STREAM, 0, false>);
}
