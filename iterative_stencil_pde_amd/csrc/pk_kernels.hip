// Launch-per-sweep, residual and setup kernels of the Jacobi engine for gfx950,
// the host-side wrappers that launch them, and the choice of persistent kernel
// instance (compiled per layout in pk_kern_*.hip from pk_persistent.h).
#include <hip/hip_runtime.h>
#include <math.h>

#include "pk_device.h"
#include "pk_launch.h"
#include "pk_shared.h"
#include "../../include/pk.h"

using namespace pkd;

namespace {

// ---- launch-per-sweep baseline and setup kernels ----------------------------
template <typename T, bool HAS_B>
__global__ void __launch_bounds__(1024) pk_sweep_launch(pk_kargs a, int src, int parity) {
    stream_sweep<T, HAS_B>(a, static_cast<const T*>(a.u[src]), static_cast<T*>(a.u[src ^ 1]), parity);
}

template <typename T, bool HAS_B>
__global__ void __launch_bounds__(1024) pk_residual_launch(pk_kargs a, int src) {
    __shared__ double s_red[16];
    const double part = stream_residual_block<T, HAS_B>(a, static_cast<const T*>(a.u[src]), s_red);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = part;
}

__global__ void __launch_bounds__(64) pk_residual_finalize(const double* partials, int grid,
                                                           double* out) {
    const double tot = sum_partials(partials, grid);
    if (threadIdx.x == 0) *out = sqrt(tot);
}

// b = (T)((h*h) * f) on every node, pitched.
template <typename T>
__global__ void __launch_bounds__(256) pk_scale_source(const T* f, T* b, int nx, int ny, int pitch,
                                                       double hh) {
    const size_t total = static_cast<size_t>(ny) * pitch;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int c = static_cast<int>(i % pitch);
        b[i] = (c < nx) ? static_cast<T>(hh * static_cast<double>(f[i])) : T(0);
    }
}

template <typename T>
const void* sweep_fn(bool has_b) {
    return has_b ? reinterpret_cast<const void*>(&pk_sweep_launch<T, true>)
                 : reinterpret_cast<const void*>(&pk_sweep_launch<T, false>);
}

}  // namespace

// ---- host-side entry points used by the runtime ------------------------------
const void* pkk_persistent_fn(int dtype, bool has_b, int layout, int rows, bool trace) {
    if (layout == PK_LAYOUT_REGISTER)
        return dtype == PK_F64 ? pkk_register_fn_f64(has_b, rows, trace) : pkk_register_fn_f32(has_b, rows, trace);
    if (layout == PK_LAYOUT_RESIDENT) return pkk_resident_fn(dtype, has_b, trace);
    // the streaming layout has no events inside its passes: one instance serves
    // traced and untraced engines
    return dtype == PK_F64 ? pkk_stream_fn_f64(has_b) : pkk_stream_fn_f32(has_b);
}

const void* pkk_sweep_fn(int dtype, bool has_b) {
    return dtype == PK_F64 ? sweep_fn<double>(has_b) : sweep_fn<float>(has_b);
}

hipError_t pkk_launch_sweep(int dtype, bool has_b, const pk_kargs& a, int threads, int src,
                            int parity, hipStream_t s) {
    const dim3 g(a.grid), b(threads);
    if (dtype == PK_F64) {
        if (has_b) hipLaunchKernelGGL((pk_sweep_launch<double, true>), g, b, 0, s, a, src, parity);
        else hipLaunchKernelGGL((pk_sweep_launch<double, false>), g, b, 0, s, a, src, parity);
    } else {
        if (has_b) hipLaunchKernelGGL((pk_sweep_launch<float, true>), g, b, 0, s, a, src, parity);
        else hipLaunchKernelGGL((pk_sweep_launch<float, false>), g, b, 0, s, a, src, parity);
    }
    return hipGetLastError();
}

hipError_t pkk_launch_residual(int dtype, bool has_b, const pk_kargs& a, int threads, int src,
                               double* out, hipStream_t s) {
    const dim3 g(a.grid), b(threads);
    if (dtype == PK_F64) {
        if (has_b) hipLaunchKernelGGL((pk_residual_launch<double, true>), g, b, 0, s, a, src);
        else hipLaunchKernelGGL((pk_residual_launch<double, false>), g, b, 0, s, a, src);
    } else {
        if (has_b) hipLaunchKernelGGL((pk_residual_launch<float, true>), g, b, 0, s, a, src);
        else hipLaunchKernelGGL((pk_residual_launch<float, false>), g, b, 0, s, a, src);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pk_residual_finalize, dim3(1), dim3(64), 0, s, a.partials, a.grid, out);
    return hipGetLastError();
}

hipError_t pkk_launch_scale_source(int dtype, const void* f, void* b, int nx, int ny, int pitch,
                                   double hh, hipStream_t s) {
    const size_t total = static_cast<size_t>(ny) * pitch;
    const size_t want = (total + 255) / 256;
    const unsigned blocks = static_cast<unsigned>(want < 4096 ? want : 4096);
    if (dtype == PK_F64)
        hipLaunchKernelGGL(pk_scale_source<double>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const double*>(f), static_cast<double*>(b), nx, ny, pitch, hh);
    else
        hipLaunchKernelGGL(pk_scale_source<float>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const float*>(f), static_cast<float*>(b), nx, ny, pitch, hh);
    return hipGetLastError();
}

// ---- scratch of the entry point that allocates nothing ------------------------
// pk_sweep_noalloc runs the launch-per-sweep kernels on the caller's buffers;
// their only scratch, one residual partial per block, lives in this array (one
// copy per GPU, held until the process ends). Host code never passes the
// array's name to a kernel: it looks the array's address up once per device
// (hipGetSymbolAddress, with that device current) and passes that address.
static __device__ __align__(256) double scratch[PK_NOALLOC_MAX_BLOCKS];

namespace {
constexpr int kMaxDevices = 64;
double* g_scratch_addr[kMaxDevices] = {};  // per device, looked up on first use
}  // namespace

hipError_t pkk_noalloc_scratch(int dev, double** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    double* p = __atomic_load_n(&g_scratch_addr[dev], __ATOMIC_ACQUIRE);
    if (!p) {
        // the caller has made `dev` current; two threads racing here store the
        // same address
        void* addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        p = static_cast<double*>(addr);
        __atomic_store_n(&g_scratch_addr[dev], p, __ATOMIC_RELEASE);
    }
    *out = p;
    return hipSuccess;
}
