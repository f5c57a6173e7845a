// Jacobi and red-black Gauss-Seidel oracle for the 5-point Poisson/Laplace
// iteration.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
// this file: only the tests, the smoke check and the CPU-baseline leg of the
// benchmark use it. It shares no code, header or constant with the HIP engine.
//
// What it computes, and where that comes from:
//   * "Persistent Kernels: Bridging GPU-CPU Execution", section "The problem
//     (another PDE solver)": Poisson's equation on the unit square, N nodes per
//     side including both ends, spacing 1/(N-1), and the 5-point update that
//     replaces each node by a quarter of its four neighbours plus the scaled
//     source term (the "Derivation" subsection gives the central differences).
//   * Same page, "Implementation details and correctness": Jacobi computes every
//     node from the previous iteration's values into a separate result matrix.
//     That is the double buffer below (A is read, B is written, then swapped).
//   * "Grid-Wide Barriers and Persistent Work Queues", section "What the barrier
//     buys": an iterative solver's convergence check is a reduction over the
//     grid. The residual below is that reduction (an L2 norm).
//
// Readings where the pages leave a step open (each one also listed in the
// design notes):
//   * Sign of the source: the problem is taken as -Lap(u) = f, so the scaled
//     source enters with a plus sign: u <- (W + E + S + N + h*h*f) / 4. With
//     f = 0 (Laplace) the term is absent.
//   * Evaluation order (the pages give the formula, not the order):
//       new = 0.25 * (((W + E) + (S + N)) + b),  b = (T)((h*h) * (double)f),
//     with W/E the left/right neighbours in the same row (fast index j) and S/N
//     the rows below/above (slow index i). IEEE round-to-nearest, no FMA
//     contraction (built with -ffp-contract=off), no flush of subnormals.
//   * Residual: R = sqrt(sum over interior cells of rho^2), with
//       rho = (((W + E) + (S + N)) + b) - 4 u,
//     every operand widened to double first and the sum accumulated in double,
//     in row-major order.
//   * Dirichlet only: the outer ring of the grid is never written.
//
// Red-black Gauss-Seidel (the iteration that page measures, same section and
// its Figure 3): in place, one iteration = first every interior node whose
// indices i and j have the same parity (red), then every interior node whose
// parities differ (black). Each node's update is the same formula as above; its
// four neighbours have the other colour, so within one half the order of the
// updates does not matter.
//
// Plain nested loops, single thread, no blocking, fusion or reordering.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

inline std::size_t at(int nx, int i, int j) {
    return static_cast<std::size_t>(i) * static_cast<std::size_t>(nx) + static_cast<std::size_t>(j);
}

// b[i][j] = (T)((h*h) * f[i][j]) on every node (ring values are never read).
template <typename T>
void scaled_source(int nx, int ny, double h, const T* F, std::vector<T>& b) {
    const double hh = h * h;
    b.assign(static_cast<std::size_t>(nx) * ny, T(0));
    for (int i = 0; i < ny; ++i)
        for (int j = 0; j < nx; ++j)
            b[at(nx, i, j)] = static_cast<T>(hh * static_cast<double>(F[at(nx, i, j)]));
}

// One Jacobi sweep: every interior node of B from the previous values in A.
template <typename T>
void sweep(int nx, int ny, const T* A, T* B, const T* b) {
    for (int i = 1; i <= ny - 2; ++i) {
        for (int j = 1; j <= nx - 2; ++j) {
            const T w = A[at(nx, i, j - 1)];
            const T e = A[at(nx, i, j + 1)];
            const T s = A[at(nx, i - 1, j)];
            const T n = A[at(nx, i + 1, j)];
            T t = (w + e) + (s + n);
            if (b) t = t + b[at(nx, i, j)];
            B[at(nx, i, j)] = T(0.25) * t;
        }
    }
}

template <typename T>
double residual(int nx, int ny, const T* A, const T* b) {
    double acc = 0.0;
    for (int i = 1; i <= ny - 2; ++i) {
        for (int j = 1; j <= nx - 2; ++j) {
            const double w = static_cast<double>(A[at(nx, i, j - 1)]);
            const double e = static_cast<double>(A[at(nx, i, j + 1)]);
            const double s = static_cast<double>(A[at(nx, i - 1, j)]);
            const double n = static_cast<double>(A[at(nx, i + 1, j)]);
            double t = (w + e) + (s + n);
            if (b) t = t + static_cast<double>(b[at(nx, i, j)]);
            const double r = t - 4.0 * static_cast<double>(A[at(nx, i, j)]);
            acc += r * r;
        }
    }
    return std::sqrt(acc);
}

// One half of a red-black iteration, in place: every interior node of colour
// `parity` ((i + j) mod 2) from the current values of its neighbours.
template <typename T>
void rb_half(int nx, int ny, T* U, const T* b, int parity) {
    for (int i = 1; i <= ny - 2; ++i) {
        for (int j = 1; j <= nx - 2; ++j) {
            if (((i + j) & 1) != parity) continue;
            const T west = U[at(nx, i, j - 1)];
            const T east = U[at(nx, i, j + 1)];
            const T south = U[at(nx, i - 1, j)];
            const T north = U[at(nx, i + 1, j)];
            T t = (west + east) + (south + north);
            if (b) t = t + b[at(nx, i, j)];
            U[at(nx, i, j)] = T(0.25) * t;
        }
    }
}

// K sweeps from U0. Before sweep k (k = 0..K) the residual is recorded once for
// every checkpoint entry equal to k (so a checkpoint of K is the final state).
// Checkpoints must be non-decreasing and lie in [0, K].
template <typename T>
int jacobi(int nx, int ny, double h, const T* U0, const T* F, int64_t K,
           const int64_t* ckpt, int nckpt, T* out, double* res_out) {
    if (nx < 3 || ny < 3 || K < 0 || !U0 || !out) return -1;
    if (nckpt < 0 || (nckpt > 0 && (!ckpt || !res_out))) return -1;
    for (int c = 0; c < nckpt; ++c) {
        if (ckpt[c] < 0 || ckpt[c] > K) return -1;
        if (c > 0 && ckpt[c] < ckpt[c - 1]) return -1;
    }
    if (F && !(h > 0.0)) return -1;
    const std::size_t cells = static_cast<std::size_t>(nx) * ny;
    std::vector<T> A(U0, U0 + cells);
    std::vector<T> B(A);  // the ring is carried by both buffers
    std::vector<T> b;
    if (F) scaled_source<T>(nx, ny, h, F, b);
    const T* bp = F ? b.data() : nullptr;
    int c = 0;
    for (int64_t k = 0;; ++k) {
        while (c < nckpt && ckpt[c] == k) res_out[c++] = residual<T>(nx, ny, A.data(), bp);
        if (k == K) break;
        sweep<T>(nx, ny, A.data(), B.data(), bp);
        A.swap(B);
    }
    std::memcpy(out, A.data(), cells * sizeof(T));
    return 0;
}

// K red-black iterations from U0 (red half, then black half, in one array);
// checkpoints as for jacobi(), counted in iterations.
template <typename T>
int rbgs(int nx, int ny, double h, const T* U0, const T* F, int64_t K,
         const int64_t* ckpt, int nckpt, T* out, double* res_out) {
    if (nx < 3 || ny < 3 || K < 0 || !U0 || !out) return -1;
    if (nckpt < 0 || (nckpt > 0 && (!ckpt || !res_out))) return -1;
    for (int c = 0; c < nckpt; ++c) {
        if (ckpt[c] < 0 || ckpt[c] > K) return -1;
        if (c > 0 && ckpt[c] < ckpt[c - 1]) return -1;
    }
    if (F && !(h > 0.0)) return -1;
    const std::size_t cells = static_cast<std::size_t>(nx) * ny;
    std::vector<T> U(U0, U0 + cells);
    std::vector<T> b;
    if (F) scaled_source<T>(nx, ny, h, F, b);
    const T* bp = F ? b.data() : nullptr;
    int c = 0;
    for (int64_t k = 0;; ++k) {
        while (c < nckpt && ckpt[c] == k) res_out[c++] = residual<T>(nx, ny, U.data(), bp);
        if (k == K) break;
        rb_half<T>(nx, ny, U.data(), bp, 0);  // red: i + j even
        rb_half<T>(nx, ny, U.data(), bp, 1);  // black: i + j odd
    }
    std::memcpy(out, U.data(), cells * sizeof(T));
    return 0;
}

template <typename T>
int residual_of(int nx, int ny, double h, const T* U, const T* F, double* r) {
    if (nx < 3 || ny < 3 || !U || !r) return -1;
    if (F && !(h > 0.0)) return -1;
    std::vector<T> b;
    if (F) scaled_source<T>(nx, ny, h, F, b);
    *r = residual<T>(nx, ny, U, F ? b.data() : nullptr);
    return 0;
}

}  // namespace

extern "C" {

int oracle_jacobi_f32(int nx, int ny, double h, const float* U0, const float* F, int64_t K,
                      const int64_t* ckpt, int nckpt, float* out, double* res_out) {
    return jacobi<float>(nx, ny, h, U0, F, K, ckpt, nckpt, out, res_out);
}

int oracle_jacobi_f64(int nx, int ny, double h, const double* U0, const double* F, int64_t K,
                      const int64_t* ckpt, int nckpt, double* out, double* res_out) {
    return jacobi<double>(nx, ny, h, U0, F, K, ckpt, nckpt, out, res_out);
}

int oracle_rbgs_f32(int nx, int ny, double h, const float* U0, const float* F, int64_t K,
                    const int64_t* ckpt, int nckpt, float* out, double* res_out) {
    return rbgs<float>(nx, ny, h, U0, F, K, ckpt, nckpt, out, res_out);
}

int oracle_rbgs_f64(int nx, int ny, double h, const double* U0, const double* F, int64_t K,
                    const int64_t* ckpt, int nckpt, double* out, double* res_out) {
    return rbgs<double>(nx, ny, h, U0, F, K, ckpt, nckpt, out, res_out);
}

int oracle_residual_f32(int nx, int ny, double h, const float* U, const float* F, double* r) {
    return residual_of<float>(nx, ny, h, U, F, r);
}

int oracle_residual_f64(int nx, int ny, double h, const double* U, const double* F, double* r) {
    return residual_of<double>(nx, ny, h, U, F, r);
}

}  // extern "C"
