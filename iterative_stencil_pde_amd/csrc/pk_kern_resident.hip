// LDS-tile instances of the persistent kernel (traced and untraced).
#include "pk_persistent.h"

using namespace pkd;

namespace {
template <typename T, bool TRACE>
const void* resident(bool has_b) {
    return has_b ? reinterpret_cast<const void*>(&pk_persistent<T, true, PK_LAYOUT_RESIDENT, 0, TRACE>)
                 : reinterpret_cast<const void*>(&pk_persistent<T, false, PK_LAYOUT_RESIDENT, 0, TRACE>);
}
}  // namespace

const void* pkk_resident_fn(int dtype, bool has_b, bool trace) {
    if (dtype == PK_F64) return trace ? resident<double, true>(has_b) : resident<double, false>(has_b);
    return trace ? resident<float, true>(has_b) : resident<float, false>(has_b);
}
