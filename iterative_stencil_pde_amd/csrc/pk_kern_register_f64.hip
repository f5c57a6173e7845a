// Register-tile instances of the persistent kernel for double (2 or 4 rows per
// wave, traced and untraced).
#include "pk_persistent.h"

using namespace pkd;

namespace {
template <int RT, bool TRACE>
const void* reg(bool has_b) {
    return has_b ? reinterpret_cast<const void*>(&pk_persistent<double, true, PK_LAYOUT_REGISTER, RT, TRACE>)
                 : reinterpret_cast<const void*>(&pk_persistent<double, false, PK_LAYOUT_REGISTER, RT, TRACE>);
}
}  // namespace

const void* pkk_register_fn_f64(bool has_b, int rows, bool trace) {
    if (rows == 2) return trace ? reg<2, true>(has_b) : reg<2, false>(has_b);
    return trace ? reg<4, true>(has_b) : reg<4, false>(has_b);
}
