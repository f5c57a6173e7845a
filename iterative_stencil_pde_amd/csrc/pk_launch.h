// Host-side launch wrappers exported by pk_kernels.hip to the runtime.
#pragma once

#include <hip/hip_runtime_api.h>

#include "pk_shared.h"

// Kernel symbol of the persistent kernel for an element type / source / layout;
// rows: rows per wave of the register layout (2 or 4, else ignored); trace: the
// instance with the tile layouts' in-loop events (PK_DBG_TRACE).
const void* pkk_persistent_fn(int dtype, bool has_b, int layout, int rows, bool trace);
// The same, per layout (one translation unit each).
const void* pkk_stream_fn_f32(bool has_b);
const void* pkk_stream_fn_f64(bool has_b);
const void* pkk_resident_fn(int dtype, bool has_b, bool trace);
const void* pkk_register_fn_f32(bool has_b, int rows, bool trace);
const void* pkk_register_fn_f64(bool has_b, int rows, bool trace);
// Kernel symbol of the one-sweep kernel (for the occupancy query).
const void* pkk_sweep_fn(int dtype, bool has_b);

// One streaming sweep u[src] -> u[src ^ 1] with a.grid blocks of `threads`;
// parity >= 0: one red-black half-sweep of that colour instead.
hipError_t pkk_launch_sweep(int dtype, bool has_b, const pk_kargs& a, int threads, int src,
                            int parity, hipStream_t s);
// Residual of u[src]: per-block partials, then one block sums them in a fixed
// order and stores sqrt(sum) at `out` (device-visible).
hipError_t pkk_launch_residual(int dtype, bool has_b, const pk_kargs& a, int threads, int src,
                               double* out, hipStream_t s);
// b = (T)((h*h) * f) on a pitched ny x pitch array.
hipError_t pkk_launch_scale_source(int dtype, const void* f, void* b, int nx, int ny, int pitch,
                                   double hh, hipStream_t s);

// Blocks the scratch of pk_sweep_noalloc holds residual partials for.
#define PK_NOALLOC_MAX_BLOCKS 1024
// Device address of that scratch on device `dev` (which must be current); looked
// up once per device and kept.
hipError_t pkk_noalloc_scratch(int dev, double** out);
