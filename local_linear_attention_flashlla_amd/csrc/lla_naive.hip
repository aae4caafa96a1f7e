// The naive causal LLA forward: the reading notes' definition (section 2.1,
// Eqs. (6)-(8)) evaluated the way section 2.2 says a direct implementation
// does it, materialising every pairwise difference z_ij = k_j - q_i
// (Theta(n^2 d) per head) and every moment matrix Sigma_i (Theta(n d^2)) in
// device memory, then solving each Sigma_i rho_i = mu_i exactly (Cholesky).
// It exists as the comparison point of the pages' peak-memory figure (Fig. 2
// of that section: FlashLLA against the naive form at d = 128) and runs in
// fp32 throughout. Four kernels, one workgroup per (query row, head):
//   naive_pairs    w_ij = exp(c q_i.k_j - max_l c q_i.k_l) and z_ij, j <= i
//   naive_moments  omega_i, mu_i = sum_j w_ij z_ij,
//                  Sigma_i = sum_j w_ij z_ij z_ij^T + lambda I
//   naive_solve    Cholesky of Sigma_i, rho_i = Sigma_i^{-1} mu_i
//   naive_output   out_i = sum_j w_ij (1 - z_ij.rho_i) v_j / sum_j w_ij (1 - z_ij.rho_i)
// (the last denominator equals omega_i - mu_i^T rho_i).

#include <hip/hip_runtime.h>

#include "lla_internal.h"

namespace lla {
namespace {

constexpr int NT = 256;  // threads per workgroup
constexpr int JC = 16;   // rows of z staged in LDS per step of the moment kernel

__device__ __forceinline__ float load_elem(const void* base, size_t idx, int dtype) {
  if (dtype == LLA_DTYPE_F32) return static_cast<const float*>(base)[idx];
  const uint32_t b = static_cast<const uint16_t*>(base)[idx];
  return __uint_as_float(b << 16);
}

struct NaiveParams {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  float* omega_out;   // optional
  float* rho_out;     // optional
  float* rowmax_out;  // optional
  int32_t* cg_iters;  // optional, written 0
  float* cg_resid;    // optional, written 0
  int dtype, BH, n;
  float lambda;
  float* Z;    // [BH][n][n][D]
  float* W;    // [BH][n][n]
  float* S;    // [BH][n][D][D]
  float* MU;   // [BH][n][D]
  float* OM;   // [BH][n]
  float* RM;   // [BH][n]
  float* RHO;  // [BH][n][D]
};

__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < NT / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

template <int D>
__global__ __launch_bounds__(NT) void naive_pairs(NaiveParams P) {
  const int i = blockIdx.x, bh = blockIdx.y, n = P.n;
  __shared__ float sq[D];
  __shared__ float red[NT / 64];
  const size_t qrow = (static_cast<size_t>(bh) * n + i) * D;
  for (int e = threadIdx.x; e < D; e += NT) sq[e] = load_elem(P.q, qrow + e, P.dtype);
  __syncthreads();
  const float c = 1.f / sqrtf(static_cast<float>(D));
  float* Wrow = P.W + (static_cast<size_t>(bh) * n + i) * n;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j <= i; j += NT) {
    const size_t krow = (static_cast<size_t>(bh) * n + j) * D;
    float s = 0.f;
    for (int e = 0; e < D; ++e) s += sq[e] * load_elem(P.k, krow + e, P.dtype);
    s *= c;
    Wrow[j] = s;
    mx = fmaxf(mx, s);
  }
  const float m = block_reduce(mx, red, true);
  // each thread rewrites the scores it wrote above
  for (int j = threadIdx.x; j <= i; j += NT) Wrow[j] = expf(Wrow[j] - m);
  if (threadIdx.x == 0) P.RM[static_cast<size_t>(bh) * n + i] = m;
  float* Zrow = P.Z + (static_cast<size_t>(bh) * n + i) * n * D;
  const size_t cnt = static_cast<size_t>(i + 1) * D;
  const size_t kbase = static_cast<size_t>(bh) * n * D;
  for (size_t e = threadIdx.x; e < cnt; e += NT)
    Zrow[e] = load_elem(P.k, kbase + e, P.dtype) - sq[e % D];
}

// Each thread owns an EB x EB block of Sigma_i (a 16 x 16 grid of blocks);
// rows of z are staged JC at a time.
template <int D>
__global__ __launch_bounds__(NT) void naive_moments(NaiveParams P) {
  constexpr int EB = D / 16;
  const int i = blockIdx.x, bh = blockIdx.y, n = P.n;
  __shared__ float sz[JC][D];
  __shared__ float sw[JC];
  const int br = threadIdx.x / 16, bc = threadIdx.x % 16;
  float acc[EB][EB];
  #pragma unroll
  for (int a = 0; a < EB; ++a)
    #pragma unroll
    for (int b = 0; b < EB; ++b) acc[a][b] = 0.f;
  float mu = 0.f, om = 0.f;  // mu: dimension threadIdx.x (< D); om: thread 0
  const float* Zrow = P.Z + (static_cast<size_t>(bh) * n + i) * n * D;
  const float* Wrow = P.W + (static_cast<size_t>(bh) * n + i) * n;
  for (int j0 = 0; j0 <= i; j0 += JC) {
    const int cnt = min(JC, i + 1 - j0);
    __syncthreads();
    for (int e = threadIdx.x; e < JC * D; e += NT) {
      const int r = e / D;
      sz[r][e % D] = r < cnt ? Zrow[static_cast<size_t>(j0) * D + e] : 0.f;
    }
    if (threadIdx.x < JC) sw[threadIdx.x] = threadIdx.x < cnt ? Wrow[j0 + threadIdx.x] : 0.f;
    __syncthreads();
    for (int r = 0; r < JC; ++r) {
      const float w = sw[r];
      float za[EB], zb[EB];
      #pragma unroll
      for (int a = 0; a < EB; ++a) {
        za[a] = sz[r][EB * br + a];
        zb[a] = sz[r][EB * bc + a];
      }
      #pragma unroll
      for (int a = 0; a < EB; ++a) {
        const float wa = w * za[a];
        #pragma unroll
        for (int b = 0; b < EB; ++b) acc[a][b] += wa * zb[b];
      }
      if (threadIdx.x < D) mu += w * sz[r][threadIdx.x];
      om += w;
    }
  }
  float* Srow = P.S + (static_cast<size_t>(bh) * n + i) * D * D;
  #pragma unroll
  for (int a = 0; a < EB; ++a)
    #pragma unroll
    for (int b = 0; b < EB; ++b) {
      const int r = EB * br + a, c = EB * bc + b;
      Srow[r * D + c] = acc[a][b] + (r == c ? P.lambda : 0.f);
    }
  const size_t row = static_cast<size_t>(bh) * n + i;
  if (threadIdx.x < D) P.MU[row * D + threadIdx.x] = mu;
  if (threadIdx.x == 0) P.OM[row] = om;
}

// Cholesky factorisation Sigma_i = L L^T in LDS (right-looking, one column
// per step), then L y = mu_i and L^T rho_i = y. A non-positive pivot (not
// possible for lambda > 0 in exact arithmetic) gives NaN, which propagates.
template <int D>
__global__ __launch_bounds__(NT) void naive_solve(NaiveParams P) {
  const int i = blockIdx.x, bh = blockIdx.y, n = P.n;
  __shared__ float A[D][D + 1];
  __shared__ float b[D];
  const size_t row = static_cast<size_t>(bh) * n + i;
  const float* Srow = P.S + row * D * D;
  for (int e = threadIdx.x; e < D * D; e += NT) A[e / D][e % D] = Srow[e];
  for (int e = threadIdx.x; e < D; e += NT) b[e] = P.MU[row * D + e];
  __syncthreads();
  for (int k = 0; k < D; ++k) {
    if (threadIdx.x == 0) A[k][k] = A[k][k] > 0.f ? sqrtf(A[k][k]) : NAN;
    __syncthreads();
    const float piv = A[k][k];
    for (int r = k + 1 + threadIdx.x; r < D; r += NT) A[r][k] /= piv;
    __syncthreads();
    const int m = D - k - 1;
    for (int e = threadIdx.x; e < m * m; e += NT) {
      const int r = k + 1 + e / m, c = k + 1 + e % m;
      if (c <= r) A[r][c] -= A[r][k] * A[c][k];
    }
    __syncthreads();
  }
  for (int k = 0; k < D; ++k) {  // L y = mu
    if (threadIdx.x == 0) b[k] /= A[k][k];
    __syncthreads();
    for (int r = k + 1 + threadIdx.x; r < D; r += NT) b[r] -= A[r][k] * b[k];
    __syncthreads();
  }
  for (int k = D - 1; k >= 0; --k) {  // L^T rho = y
    if (threadIdx.x == 0) b[k] /= A[k][k];
    __syncthreads();
    for (int r = threadIdx.x; r < k; r += NT) b[r] -= A[k][r] * b[k];
    __syncthreads();
  }
  for (int e = threadIdx.x; e < D; e += NT) P.RHO[row * D + e] = b[e];
}

template <int D>
__global__ __launch_bounds__(NT) void naive_output(NaiveParams P) {
  constexpr int G = NT / D;  // key subsets per output dimension
  const int i = blockIdx.x, bh = blockIdx.y, n = P.n;
  __shared__ float srho[D];
  __shared__ float sa[NT];
  __shared__ float red[NT / 64];
  __shared__ float part[G][D];
  const size_t row = static_cast<size_t>(bh) * n + i;
  for (int e = threadIdx.x; e < D; e += NT) srho[e] = P.RHO[row * D + e];
  __syncthreads();
  const float* Zrow = P.Z + row * n * D;
  const float* Wrow = P.W + row * n;
  const size_t vbase = static_cast<size_t>(bh) * n * D;
  const int dim = threadIdx.x % D, sub = threadIdx.x / D;
  float acc = 0.f, den = 0.f;
  for (int j0 = 0; j0 <= i; j0 += NT) {
    const int j = j0 + threadIdx.x;
    float a = 0.f;
    if (j <= i) {
      const float* z = Zrow + static_cast<size_t>(j) * D;
      float zr = 0.f;
      for (int e = 0; e < D; ++e) zr += z[e] * srho[e];
      a = Wrow[j] * (1.f - zr);
    }
    den += a;
    __syncthreads();
    sa[threadIdx.x] = a;
    __syncthreads();
    const int cnt = min(NT, i + 1 - j0);
    for (int r = sub; r < cnt; r += G)
      acc += sa[r] * load_elem(P.v, vbase + static_cast<size_t>(j0 + r) * D + dim, P.dtype);
  }
  const float tot = block_reduce(den, red, false);
  part[sub][dim] = acc;
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += part[g][threadIdx.x];
    P.out[row * D + threadIdx.x] = s / tot;
    if (P.rho_out) P.rho_out[row * D + threadIdx.x] = srho[threadIdx.x];
  }
  if (threadIdx.x == 0) {
    if (P.omega_out) P.omega_out[row] = P.OM[row];
    if (P.rowmax_out) P.rowmax_out[row] = P.RM[row];
    if (P.cg_iters) P.cg_iters[row] = 0;
    if (P.cg_resid) P.cg_resid[row] = 0.f;
  }
}

struct NaiveLayout {
  size_t z, w, s, mu, om, rm, rho, total;
};

size_t align256n(size_t x) { return (x + 255) & ~size_t(255); }

NaiveLayout naive_layout(int BH, int n, int d) {
  const size_t rows = static_cast<size_t>(BH) * n;
  NaiveLayout L;
  size_t p = 0;
  L.z = p;   p += align256n(rows * n * d * sizeof(float));
  L.w = p;   p += align256n(rows * n * sizeof(float));
  L.s = p;   p += align256n(rows * d * d * sizeof(float));
  L.mu = p;  p += align256n(rows * d * sizeof(float));
  L.om = p;  p += align256n(rows * sizeof(float));
  L.rm = p;  p += align256n(rows * sizeof(float));
  L.rho = p; p += align256n(rows * d * sizeof(float));
  L.total = p;
  return L;
}

template <int D>
hipError_t launch_naive_d(NaiveParams P, const FwdParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.n), static_cast<unsigned>(p.BH));
  hipLaunchKernelGGL(naive_pairs<D>, grid, dim3(NT), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_main_begin && (e = hipEventRecord(p.ev_main_begin, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(naive_moments<D>, grid, dim3(NT), 0, stream, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.ev_main_end && (e = hipEventRecord(p.ev_main_end, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(naive_solve<D>, grid, dim3(NT), 0, stream, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(naive_output<D>, grid, dim3(NT), 0, stream, P);
  return hipGetLastError();
}

}  // namespace

size_t naive_workspace_bytes(int BH, int n, int d) { return naive_layout(BH, n, d).total; }

hipError_t launch_naive(const FwdParams& p, hipStream_t stream) {
  const NaiveLayout L = naive_layout(p.BH, p.n, p.d);
  char* base = static_cast<char*>(p.workspace);
  NaiveParams P{};
  P.q = p.q; P.k = p.k; P.v = p.v; P.out = p.out;
  P.omega_out = p.omega; P.rho_out = p.rho; P.rowmax_out = p.rowmax;
  P.cg_iters = p.cg_iters; P.cg_resid = p.cg_resid;
  P.dtype = p.dtype; P.BH = p.BH; P.n = p.n; P.lambda = p.lambda;
  P.Z = reinterpret_cast<float*>(base + L.z);
  P.W = reinterpret_cast<float*>(base + L.w);
  P.S = reinterpret_cast<float*>(base + L.s);
  P.MU = reinterpret_cast<float*>(base + L.mu);
  P.OM = reinterpret_cast<float*>(base + L.om);
  P.RM = reinterpret_cast<float*>(base + L.rm);
  P.RHO = reinterpret_cast<float*>(base + L.rho);
  switch (p.d) {
    case 16: return launch_naive_d<16>(P, p, stream);
    case 32: return launch_naive_d<32>(P, p, stream);
    case 64: return launch_naive_d<64>(P, p, stream);
    case 128: return launch_naive_d<128>(P, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lla
