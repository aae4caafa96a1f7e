// fp32 vector-ALU kernels for the causal LLA forward and backward passes.
//
// In the forward, one workgroup of 256 threads owns a block of 4, 8, 16 or 32
// consecutive query rows of one (batch, head) and runs all three phases of the
// blocked forward of "Local Linear Attention: reading notes" (section 2.2,
// Algorithm 1) for it:
//   1. scan key tiles with an online row max -> omega_i, mu~_i (Eqs. (10)-(11))
//   2. matrix-free CG, one key-tile sweep per iteration for the Gram product
//      (Eq. (12), centred at kbar_i = mu~_i / omega_i; see include/lla.h)
//   3. scan key/value tiles -> out_i = sum_j w_ij (1 - (k_j - kbar_i)^T rho) v_j
//      / sum_j w_ij (1 - (k_j - kbar_i)^T rho)
// Per-query CG state lives in registers (x, r, kbar, accumulators) and LDS
// (q, p); the weights exist only as a rows x tile-keys tile in LDS. The next
// key (and value) tile is loaded into registers while the current one is used.
//
// Thread roles (forward): the LPR = 8, 16, 32 or 64 lanes of a row group serve one
// query row (row reductions are xor-shuffles within the group). For score
// tiles a lane computes keys l and l + LPR of a 2 LPR-key tile; for d-vectors
// it owns float4 chunks and a slice of the tile's keys (struct Lanes below).
// The backward uses the same layouts.
//
// These kernels are the fp32 path (fp32 inputs must not be rounded to a 16-bit
// matrix type) and the reference GPU path for bf16 inputs.

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "lla_internal.h"
#include "../../include/lla.h"

namespace lla {
namespace {

constexpr int VT = 256;  // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float load_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

__device__ __forceinline__ float4 load4(const float* p, size_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
__device__ __forceinline__ float4 load4(const uint16_t* p, size_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

__device__ __forceinline__ float row_sum8(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  return v;
}
__device__ __forceinline__ float row_max8(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  return v;
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c) {
  return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}

// Load rows [r0, r0 + rows) of a [n][D] matrix into LDS (row stride LD
// floats), zero-filling rows at or beyond `rend`.
template <int D, int LD, typename Tin>
__device__ __forceinline__ void stage_rows(float* dst, const Tin* src, int r0, int rows,
                                           int rend) {
  constexpr int NC = D / 4;
  for (int e = threadIdx.x; e < rows * NC; e += VT) {
    const int r = e / NC, c = (e % NC) * 4;
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + r < rend) val = load4(src, static_cast<size_t>(r0 + r) * D + c);
    *reinterpret_cast<float4*>(dst + r * LD + c) = val;
  }
}

// Lane layout of the forward. LPR lanes serve one query row, so a workgroup
// holds VQ = VT / LPR rows and a key tile VK = 2 LPR keys (two scores per
// lane). A d-vector is split into CL = min(d / 4, LPR) float4 columns and
// S = LPR / CL key slices: lane l of a row owns chunks (l % CL) + CL u and
// adds up keys l / CL + S m of each tile; the slices are summed once per
// sweep. Small problems take more lanes per row (more workgroups, fewer and
// wider tiles per sweep); large ones fewer (keys re-read by fewer blocks).
template <int D, int LPR>
struct Lanes {
  static constexpr int VQ = VT / LPR;
  static constexpr int VK = 2 * LPR;
  static constexpr int NC = D / 4;
  static constexpr int CL = NC < LPR ? NC : LPR;
  static constexpr int S = LPR / CL;
  static constexpr int YC = NC / CL;
};

// sum / max over the W lanes of a row group (W a power of two <= 64)
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  #pragma unroll
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o);
  return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
  #pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// sum of a chunk over the key slices (lanes CL, 2 CL, ... apart)
template <int CL, int LPR>
__device__ __forceinline__ float4 slice_sum(float4 a) {
  #pragma unroll
  for (int o = CL; o < LPR; o <<= 1) {
    a.x += __shfl_xor(a.x, o);
    a.y += __shfl_xor(a.y, o);
    a.z += __shfl_xor(a.z, o);
    a.w += __shfl_xor(a.w, o);
  }
  return a;
}

// A tile of ROWS rows of a [n][D] matrix held in registers between its global
// loads and its LDS store, so that the next tile's loads are in flight while
// the current one is used (float4 e = threadIdx.x + VT u of the tile).
template <int D, int ROWS>
struct TileRegs {
  static constexpr int NC = D / 4;
  static constexpr int NU = ROWS > 0 ? (ROWS * NC + VT - 1) / VT : 1;  // (1: unused)
  float4 v[NU];
  // rows [r0, r0 + ROWS), zero at or beyond rend
  template <typename Tin>
  __device__ __forceinline__ void load(const Tin* src, int r0, int rend) {
    #pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = static_cast<int>(threadIdx.x) + VT * u;
      const int r = e / NC, c = (e % NC) * 4;
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < ROWS * NC && r0 + r < rend) v[u] = load4(src, static_cast<size_t>(r0 + r) * D + c);
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(float* dst) const {
    #pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = static_cast<int>(threadIdx.x) + VT * u;
      if (e < ROWS * NC) *reinterpret_cast<float4*>(dst + (e / NC) * LD + (e % NC) * 4) = v[u];
    }
  }
};

// ls > 0: the block's score weights are kept in dynamic LDS (row r, key j at
// r ls + j), written in phase 1 and read by every later sweep in place of the
// q . k products and exponentials (the same weights up to the rounding of the
// score's scaling, which the recomputing form may fuse into the exponent's
// subtraction).
template <int D, typename Tin, int LPR>
__global__ __launch_bounds__(VT) void lla_valu_kernel(FwdParams P, int ls) {
  using L = Lanes<D, LPR>;
  constexpr int BQ = L::VQ, BKV = L::VK, CL = L::CL, S = L::S, YC = L::YC;
  constexpr int LD = D + 4;   // padded LDS row stride (floats)
  constexpr int LW = BKV + 1;  // row stride of the weight tile
  __shared__ __align__(16) float sQ[BQ * LD];   // q rows of the block
  __shared__ __align__(16) float sP[BQ * LD];   // p (phase 2) / rho (phase 3)
  __shared__ __align__(16) float sK[BKV * LD];  // key tile
  __shared__ __align__(16) float sV[BKV * LD];  // value tile (phase 3)
  __shared__ float sW[BQ * LW];                 // weight-derived tile
  __shared__ int sAny;
  extern __shared__ float sS[];                 // cached weights (ls > 0)

  const int tid = threadIdx.x;
  const int row = tid / LPR;
  const int ln = tid % LPR;
  const int cl = ln % CL, sl = ln / CL;
  const int nqb = (P.n + BQ - 1) / BQ;
  const int blk = blockIdx.x;
  const int qb = nqb - 1 - blk / P.BH;  // longest causal prefix first
  const int bh = blk % P.BH;
  const int i0 = qb * BQ;
  const int nq = min(BQ, P.n - i0);
  const int kend = i0 + nq;           // keys 0 .. kend-1 are visible to the block
  const int qi = i0 + row;            // this thread's query row
  const bool valid = row < nq;
  const size_t base = static_cast<size_t>(bh) * P.n * D;
  const Tin* Q = static_cast<const Tin*>(P.q) + base;
  const Tin* K = static_cast<const Tin*>(P.k) + base;
  const Tin* V = static_cast<const Tin*>(P.v) + base;
  const float sc2 = kLog2e / sqrtf(static_cast<float>(D));  // scores in log2 units
  const float lam = P.lambda;
  const float* qrow = sQ + row * LD;
  const float* prow = sP + row * LD;
  const bool cached = ls > 0;  // uniform
  float* srow = sS + row * ls;

  // Small blocks (more lanes per row) are latency-bound: they load the next
  // tile into registers while the current one is used. With 32 rows per
  // block the registers are better spent on the block's own state.
  constexpr bool PREFETCH = LPR > 8;
  stage_rows<D, LD>(sQ, Q, i0, BQ, kend);
  TileRegs<D, PREFETCH ? BKV : 0> kpre;
  auto first_keys = [&]() __attribute__((always_inline)) {
    if constexpr (PREFETCH) kpre.load(K, 0, kend);
  };
  // key tile kt into sK (between two barriers)
  auto next_keys = [&](int kt) __attribute__((always_inline)) {
    __syncthreads();
    if constexpr (PREFETCH) {
      kpre.template store<LD>(sK);
      if (kt + BKV < kend) kpre.load(K, kt + BKV, kend);
    } else {
      stage_rows<D, LD>(sK, K, kt, BKV, kend);
    }
    __syncthreads();
  };
  // acc[u] += sum over this lane's slice of the tile's keys of sW[row][kk] X[kk][chunk u]
  auto tile_product = [&](float4 (&a)[YC], const float* X) __attribute__((always_inline)) {
    #pragma unroll
    for (int u = 0; u < YC; ++u) {
      const int c = (cl + CL * u) * 4;
      float4 t = a[u];
      #pragma unroll
      for (int m = 0; m < BKV / S; ++m) {
        const int kk = sl + S * m;
        t = fma4(sW[row * LW + kk], *reinterpret_cast<const float4*>(X + kk * LD + c), t);
      }
      a[u] = t;
    }
  };

  // ---------------- phase 1: online max, omega, mu~ ----------------
  float m2 = -INFINITY;  // running row max (log2 units)
  float om = 0.f;
  float4 acc[YC];
  for (int u = 0; u < YC; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);

  first_keys();
  for (int kt = 0; kt < kend; kt += BKV) {
    next_keys(kt);
    float s[2];
    float tmax = -INFINITY;
    for (int u = 0; u < 2; ++u) {
      const int kc = ln + LPR * u;
      const int j = kt + kc;
      float dsum = 0.f;
      for (int c = 0; c < D; c += 4)
        dsum += dot4(*reinterpret_cast<const float4*>(qrow + c),
                     *reinterpret_cast<const float4*>(sK + kc * LD + c));
      s[u] = (valid && j <= qi) ? dsum * sc2 : -INFINITY;
      tmax = fmaxf(tmax, s[u]);
      if (cached) srow[j] = s[u];
    }
    tmax = group_max<LPR>(tmax);
    const float mnew = fmaxf(m2, tmax);
    const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m2 - mnew);
    float psum = 0.f;
    for (int u = 0; u < 2; ++u) {
      const float w = (s[u] == -INFINITY) ? 0.f : exp2f(s[u] - mnew);
      sW[row * LW + ln + LPR * u] = w;
      psum += w;
    }
    om = om * alpha + group_sum<LPR>(psum);
    m2 = mnew;
    for (int u = 0; u < YC; ++u) {
      acc[u].x *= alpha; acc[u].y *= alpha; acc[u].z *= alpha; acc[u].w *= alpha;
    }
    __syncthreads();
    tile_product(acc, sK);
  }
  for (int u = 0; u < YC; ++u) acc[u] = slice_sum<CL, LPR>(acc[u]);
  // scores -> weights against the final row max (each lane its own keys)
  if (cached) {
    for (int j = ln; j < kend; j += LPR) {
      const float sj = srow[j];
      srow[j] = (sj == -INFINITY) ? 0.f : exp2f(sj - m2);
    }
  }

  // ------------- CG set-up on the mean-centred system ----------------
  // kbar = mu~ / omega; mu = mu~ - omega q = omega (kbar - q); x0 = 0, r0 = p0 = mu.
  // Every slice holds the row's chunks; dot products sum over the CL chunk lanes.
  float4 kb[YC], x[YC], r[YC];
  float rr = 0.f, kp = 0.f;
  const float inv_om = valid ? 1.f / om : 0.f;
  for (int u = 0; u < YC; ++u) {
    const int c = (cl + CL * u) * 4;
    kb[u] = x[u] = r[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
      const float4 qv = *reinterpret_cast<const float4*>(qrow + c);
      const float4 a = acc[u];
      if (P.rho_in) {
        // rho supplied: no solve; the output scan is centred at q, which is
        // Eq. (8) as printed
        kb[u] = qv;
        x[u] = *reinterpret_cast<const float4*>(P.rho_in + (static_cast<size_t>(bh) * P.n + qi) * D + c);
        continue;
      }
      kb[u] = make_float4(a.x * inv_om, a.y * inv_om, a.z * inv_om, a.w * inv_om);
      r[u] = make_float4(a.x - om * qv.x, a.y - om * qv.y, a.z - om * qv.z, a.w - om * qv.w);
      rr += dot4(r[u], r[u]);
      kp += dot4(kb[u], r[u]);
    }
  }
  __syncthreads();  // sP is free (phase 1 never touched it) but keep LDS phases apart
  if (sl == 0) {
    for (int u = 0; u < YC; ++u)
      *reinterpret_cast<float4*>(sP + row * LD + (cl + CL * u) * 4) = r[u];
  }
  rr = group_sum<CL>(rr);
  kp = group_sum<CL>(kp);
  const float r0 = sqrtf(rr);
  const float stop_at = P.cg_rel_tol * r0;
  bool active = valid && rr > 0.f && P.cg_max_iters > 0;
  int iters = 0;

  // ---------------- phase 2: matrix-free CG ----------------
  for (int it = 0; it < P.cg_max_iters; ++it) {
    if (tid == 0) sAny = 0;
    __syncthreads();
    if (active && ln == 0) sAny = 1;
    __syncthreads();
    if (!sAny) break;
    // Y = sum_j w_ij k_j ((k_j - kbar) . p) over the causal prefix
    float usum = 0.f;
    for (int u = 0; u < YC; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    first_keys();
    for (int kt = 0; kt < kend; kt += BKV) {
      next_keys(kt);
      for (int u = 0; u < 2; ++u) {
        const int kc = ln + LPR * u;
        const int j = kt + kc;
        float ds = 0.f, dt = 0.f;
        if (cached) {
          for (int c = 0; c < D; c += 4)
            dt += dot4(*reinterpret_cast<const float4*>(prow + c),
                       *reinterpret_cast<const float4*>(sK + kc * LD + c));
        } else {
          for (int c = 0; c < D; c += 4) {
            const float4 kv = *reinterpret_cast<const float4*>(sK + kc * LD + c);
            ds += dot4(*reinterpret_cast<const float4*>(qrow + c), kv);
            dt += dot4(*reinterpret_cast<const float4*>(prow + c), kv);
          }
        }
        float U = 0.f;
        if (valid && j <= qi) U = (cached ? srow[j] : exp2f(ds * sc2 - m2)) * (dt - kp);
        sW[row * LW + kc] = U;
        usum += U;
      }
      __syncthreads();
      tile_product(acc, sK);
    }
    usum = group_sum<LPR>(usum);
    for (int u = 0; u < YC; ++u) acc[u] = slice_sum<CL, LPR>(acc[u]);
    // Sigma_c p = Y - (sum_j U_ij) kbar + lambda p; then the CG step.
    float pAp = 0.f;
    float4 Ap[YC], pv[YC];
    for (int u = 0; u < YC; ++u) {
      const int c = (cl + CL * u) * 4;
      pv[u] = *reinterpret_cast<const float4*>(prow + c);
      const float4 a = acc[u];
      Ap[u] = make_float4(a.x - usum * kb[u].x + lam * pv[u].x, a.y - usum * kb[u].y + lam * pv[u].y,
                          a.z - usum * kb[u].z + lam * pv[u].z, a.w - usum * kb[u].w + lam * pv[u].w);
      pAp += dot4(pv[u], Ap[u]);
    }
    pAp = group_sum<CL>(pAp);
    bool step = active && pAp > 0.f;
    if (active && !step) active = false;  // breakdown
    float rrn = 0.f;
    const float al = step ? rr / pAp : 0.f;
    for (int u = 0; u < YC; ++u) {
      if (step) {
        x[u] = fma4(al, pv[u], x[u]);
        r[u] = fma4(-al, Ap[u], r[u]);
      }
      rrn += dot4(r[u], r[u]);
    }
    rrn = group_sum<CL>(rrn);
    float kpn = 0.f;
    if (step) {
      ++iters;
      if (sqrtf(rrn) <= stop_at || rrn == 0.f) {
        active = false;
      } else {
        const float be = rrn / rr;
        for (int u = 0; u < YC; ++u) {
          pv[u] = fma4(be, pv[u], r[u]);
          // (every lane of the row has read p above: one wave holds the row)
          if (sl == 0) *reinterpret_cast<float4*>(sP + row * LD + (cl + CL * u) * 4) = pv[u];
          kpn += dot4(kb[u], pv[u]);
        }
      }
      rr = rrn;
    }
    kpn = group_sum<CL>(kpn);
    if (active) kp = kpn;
    __syncthreads();
  }

  // ---------------- phase 3: output scan ----------------
  // a_ij = w_ij (1 - (k_j - kbar) . rho_c); out_i = sum_j a_ij v_j / sum_j a_ij
  __syncthreads();
  float kr = 0.f, qr = 0.f;
  for (int u = 0; u < YC; ++u) {
    const int c = (cl + CL * u) * 4;
    if (sl == 0) *reinterpret_cast<float4*>(sP + row * LD + c) = x[u];
    kr += dot4(kb[u], x[u]);
    qr += dot4(*reinterpret_cast<const float4*>(qrow + c), x[u]);
    acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  kr = group_sum<CL>(kr);
  qr = group_sum<CL>(qr);
  float den = 0.f;
  TileRegs<D, PREFETCH ? BKV : 0> vpre;
  if constexpr (PREFETCH) {
    kpre.load(K, 0, kend);
    vpre.load(V, 0, kend);
  }
  for (int kt = 0; kt < kend; kt += BKV) {
    __syncthreads();
    if constexpr (PREFETCH) {
      kpre.template store<LD>(sK);
      vpre.template store<LD>(sV);
      if (kt + BKV < kend) {
        kpre.load(K, kt + BKV, kend);
        vpre.load(V, kt + BKV, kend);
      }
    } else {
      stage_rows<D, LD>(sK, K, kt, BKV, kend);
      stage_rows<D, LD>(sV, V, kt, BKV, kend);
    }
    __syncthreads();
    for (int u = 0; u < 2; ++u) {
      const int kc = ln + LPR * u;
      const int j = kt + kc;
      float ds = 0.f, dr = 0.f;
      if (cached) {
        for (int c = 0; c < D; c += 4)
          dr += dot4(*reinterpret_cast<const float4*>(prow + c),
                     *reinterpret_cast<const float4*>(sK + kc * LD + c));
      } else {
        for (int c = 0; c < D; c += 4) {
          const float4 kv = *reinterpret_cast<const float4*>(sK + kc * LD + c);
          ds += dot4(*reinterpret_cast<const float4*>(qrow + c), kv);
          dr += dot4(*reinterpret_cast<const float4*>(prow + c), kv);
        }
      }
      float a = 0.f;
      if (valid && j <= qi) a = (cached ? srow[j] : exp2f(ds * sc2 - m2)) * (1.f - (dr - kr));
      sW[row * LW + kc] = a;
      den += a;
    }
    __syncthreads();
    tile_product(acc, sV);
  }
  den = group_sum<LPR>(den);
  for (int u = 0; u < YC; ++u) acc[u] = slice_sum<CL, LPR>(acc[u]);
  if (!valid) return;
  const size_t orow = static_cast<size_t>(bh) * P.n + qi;
  const float inv_den = 1.f / den;
  // the pages' rho_i = Sigma_i^{-1} mu_i = rho_c / (1 + (kbar - q) . rho_c)
  const float rs = 1.f / (1.f + (kr - qr));
  if (sl == 0) {
    for (int u = 0; u < YC; ++u) {
      const int c = (cl + CL * u) * 4;
      const float4 o = acc[u];
      *reinterpret_cast<float4*>(P.out + orow * D + c) =
          make_float4(o.x * inv_den, o.y * inv_den, o.z * inv_den, o.w * inv_den);
      if (P.rho)
        *reinterpret_cast<float4*>(P.rho + orow * D + c) =
            make_float4(x[u].x * rs, x[u].y * rs, x[u].z * rs, x[u].w * rs);
      if (P.rho_c) *reinterpret_cast<float4*>(P.rho_c + orow * D + c) = x[u];
    }
  }
  if (ln == 0) {
    if (P.omega) P.omega[orow] = om;
    if (P.rowmax) P.rowmax[orow] = m2 * kLn2;
    if (P.cg_iters) P.cg_iters[orow] = iters;
    if (P.cg_resid) P.cg_resid[orow] = r0 > 0.f ? sqrtf(rr) / r0 : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Gradient of the forward above (fp32 arithmetic, any d in {16,32,64,128},
// fp32 or bf16 inputs): dq, dk, dv of sum(dout * out). One workgroup per block
// of 32, 16 or 8 queries, the lane layouts and the weight cache of the forward
// (the same choice per launch). The gradient is implicit
// differentiation of Eqs. (6)-(8) of "Local Linear Attention: reading notes"
// (section 2.1) in the form centred at kbar, as in the matrix-core backward:
//   h = C^T g,  adjoint CG  Sigma_c y = h  (the forward's CG loop on h),
//   e_j = (g.v_j - g.vbar)/omega - (k_j - kbar).y,  A_j = 1 - (k_j - kbar).rho_c,
//   dL/ds_j = w_j (A_j e_j + tau),  tau = h.rho_c/omega - y.(kbar - q),
//   and the max's share at the maximising key j* (its row sum, -lambda y.rho_c);
//   dq = c sum_j dL/ds_j k_j + omega y;
//   dk_j += c dL/ds_j q - w_j (A_j y + e_j rho_c);  dv_j += (w_j A_j / omega) g.
// Phase 1 is the forward's, operation for operation, so the row max and kbar
// (and with them the forward's rho_c) are reproduced exactly. dk and dv are
// reduced over the block's queries in LDS per key tile and added to the
// zero-filled outputs with fp32 atomics.
template <int D, typename Tin, int LPR>
__global__ __launch_bounds__(VT) void lla_valu_bwd_kernel(BwdParams P, int ls) {
  using L = Lanes<D, LPR>;
  constexpr int BQ = L::VQ, BKV = L::VK, NC = L::NC, CL = L::CL, S = L::S, YC = L::YC;
  constexpr int LD = D + 4;
  constexpr int LW = BKV + 1;
  // as in the forward; at d = 128 the two tiles' registers would spill
  constexpr bool PREFETCH = LPR > 8 && D <= 64;
  __shared__ __align__(16) float sQ[BQ * LD];   // q rows
  __shared__ __align__(16) float sG[BQ * LD];   // dout rows
  __shared__ __align__(16) float sP[BQ * LD];   // CG direction, then rho_c
  __shared__ __align__(16) float sY[BQ * LD];   // y
  __shared__ __align__(16) float sK[BKV * LD];
  __shared__ __align__(16) float sV[BKV * LD];
  __shared__ float sW[BQ * LW];                 // weight tile / dL/ds
  __shared__ float sA[BQ * LW];                 // c dL/ds with the max's share (dk)
  __shared__ float sB[BQ * LW];                 // -w A
  __shared__ float sE[BQ * LW];                 // -w e
  __shared__ float sOm[BQ];
  __shared__ int sAny;
  extern __shared__ float sS[];                 // cached weights (ls > 0), as in the forward

  const int tid = threadIdx.x;
  const int row = tid / LPR;
  const int ln = tid % LPR;
  const int cl = ln % CL, sl = ln / CL;
  const int nqb = (P.n + BQ - 1) / BQ;
  const int blk = blockIdx.x;
  const int qb = nqb - 1 - blk / P.BH;
  const int bh = blk % P.BH;
  const int i0 = qb * BQ;
  const int nq = min(BQ, P.n - i0);
  const int kend = i0 + nq;
  const int qi = i0 + row;
  const bool valid = row < nq;
  const size_t base = static_cast<size_t>(bh) * P.n * D;
  const Tin* Q = static_cast<const Tin*>(P.q) + base;
  const Tin* K = static_cast<const Tin*>(P.k) + base;
  const Tin* V = static_cast<const Tin*>(P.v) + base;
  const float sc2 = kLog2e / sqrtf(static_cast<float>(D));
  const float cs = 1.f / sqrtf(static_cast<float>(D));
  const float lam = P.lambda;
  const size_t orow = base + static_cast<size_t>(valid ? qi : i0) * D;
  const float* qrow = sQ + row * LD;
  const float* grow = sG + row * LD;
  const float* prow = sP + row * LD;
  const float* yrow = sY + row * LD;
  const bool cached = ls > 0;  // uniform
  float* srow = sS + row * ls;

  stage_rows<D, LD>(sQ, Q, i0, BQ, kend);
  for (int e = tid; e < BQ * NC; e += VT) {
    const int r = e / NC, c = (e % NC) * 4;
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < nq) val = *reinterpret_cast<const float4*>(P.dout + base + static_cast<size_t>(i0 + r) * D + c);
    *reinterpret_cast<float4*>(sG + r * LD + c) = val;
  }
  TileRegs<D, PREFETCH ? BKV : 0> kpre, vpre;
  // the first tile of a sweep over K (and V)
  auto first = [&](bool with_v) __attribute__((always_inline)) {
    if constexpr (PREFETCH) {
      kpre.load(K, 0, kend);
      if (with_v) vpre.load(V, 0, kend);
    }
  };
  // tile kt into sK (and sV) between two barriers, the next tile's loads issued
  auto next = [&](int kt, bool with_v) __attribute__((always_inline)) {
    __syncthreads();
    if constexpr (PREFETCH) {
      kpre.template store<LD>(sK);
      if (with_v) vpre.template store<LD>(sV);
      if (kt + BKV < kend) {
        kpre.load(K, kt + BKV, kend);
        if (with_v) vpre.load(V, kt + BKV, kend);
      }
    } else {
      stage_rows<D, LD>(sK, K, kt, BKV, kend);
      if (with_v) stage_rows<D, LD>(sV, V, kt, BKV, kend);
    }
    __syncthreads();
  };
  // acc[u] += sum over this lane's slice of the tile's keys of sW[row][kk] sK[kk][chunk u]
  auto tile_product = [&](float4 (&a)[YC]) __attribute__((always_inline)) {
    #pragma unroll
    for (int u = 0; u < YC; ++u) {
      const int c = (cl + CL * u) * 4;
      float4 t = a[u];
      for (int m = 0; m < BKV / S; ++m) {
        const int kk = sl + S * m;
        t = fma4(sW[row * LW + kk], *reinterpret_cast<const float4*>(sK + kk * LD + c), t);
      }
      a[u] = t;
    }
  };

  // ---------------- phase 1 (the forward's): row max, omega, mu~ ----------------
  float m2 = -INFINITY;
  float om = 0.f;
  float4 acc[YC];
  for (int u = 0; u < YC; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  float bestv = -INFINITY;
  int bestj = valid ? qi : 0;  // the maximising key (ties: the smaller index)
  first(false);
  for (int kt = 0; kt < kend; kt += BKV) {
    next(kt, false);
    float s[2];
    float tmax = -INFINITY;
    for (int u = 0; u < 2; ++u) {
      const int kc = ln + LPR * u;
      const int j = kt + kc;
      float dsum = 0.f;
      for (int c = 0; c < D; c += 4)
        dsum += dot4(*reinterpret_cast<const float4*>(qrow + c),
                     *reinterpret_cast<const float4*>(sK + kc * LD + c));
      s[u] = (valid && j <= qi) ? dsum * sc2 : -INFINITY;
      tmax = fmaxf(tmax, s[u]);
      if (cached) srow[j] = s[u];
      if (s[u] > bestv || (s[u] == bestv && s[u] != -INFINITY && j < bestj)) {
        bestv = s[u];
        bestj = j;
      }
    }
    tmax = group_max<LPR>(tmax);
    const float mnew = fmaxf(m2, tmax);
    const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m2 - mnew);
    float psum = 0.f;
    for (int u = 0; u < 2; ++u) {
      const float w = (s[u] == -INFINITY) ? 0.f : exp2f(s[u] - mnew);
      sW[row * LW + ln + LPR * u] = w;
      psum += w;
    }
    om = om * alpha + group_sum<LPR>(psum);
    m2 = mnew;
    for (int u = 0; u < YC; ++u) {
      acc[u].x *= alpha; acc[u].y *= alpha; acc[u].z *= alpha; acc[u].w *= alpha;
    }
    __syncthreads();
    tile_product(acc);
  }
  for (int u = 0; u < YC; ++u) acc[u] = slice_sum<CL, LPR>(acc[u]);
  if (cached) {
    for (int j = ln; j < kend; j += LPR) {
      const float sj = srow[j];
      srow[j] = (sj == -INFINITY) ? 0.f : exp2f(sj - m2);
    }
  }
  // the row's maximising key: larger score, then smaller index, over the row's lanes
  #pragma unroll
  for (int o = 1; o < LPR; o <<= 1) {
    const float ov = __shfl_xor(bestv, o);
    const int oj = __shfl_xor(bestj, o);
    if (ov > bestv || (ov == bestv && oj < bestj)) {
      bestv = ov;
      bestj = oj;
    }
  }
  const float inv_om = valid ? 1.f / om : 0.f;
  float4 kb[YC], qv[YC];
  float gb = 0.f;
  for (int u = 0; u < YC; ++u) {
    const int c = (cl + CL * u) * 4;
    kb[u] = qv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
      const float4 a = acc[u];
      kb[u] = make_float4(a.x * inv_om, a.y * inv_om, a.z * inv_om, a.w * inv_om);
      qv[u] = *reinterpret_cast<const float4*>(qrow + c);
      gb += dot4(*reinterpret_cast<const float4*>(grow + c), *reinterpret_cast<const float4*>(P.out + orow + c));
    }
  }
  gb = group_sum<CL>(gb);

  // w_ij (final row max) of key j of the tile (lane's key kc): cached, or from q . k
  auto weight = [&](int kc, int j) __attribute__((always_inline)) -> float {
    if (!(valid && j <= qi)) return 0.f;
    if (cached) return srow[j];
    float ds = 0.f;
    for (int c = 0; c < D; c += 4)
      ds += dot4(*reinterpret_cast<const float4*>(qrow + c),
                 *reinterpret_cast<const float4*>(sK + kc * LD + c));
    return exp2f(ds * sc2 - m2);
  };
  // the same weight, with the key's products with rows a and b (nb of them)
  // formed in the one pass over the key that also forms q . k if needed
  auto weight_dots = [&](int kc, int j, int nb, const float* a, float& da, const float* b,
                         float& db) __attribute__((always_inline)) -> float {
    float ds = 0.f;
    da = db = 0.f;
    // (two loops, so that neither carries a branch: one inside the loop keeps
    // the compiler from batching the loads across its iterations)
    if (cached) {
      for (int c = 0; c < D; c += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(sK + kc * LD + c);
        da += dot4(*reinterpret_cast<const float4*>(a + c), kv);
        if (nb > 1) db += dot4(*reinterpret_cast<const float4*>(b + c), kv);
      }
    } else {
      for (int c = 0; c < D; c += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(sK + kc * LD + c);
        ds += dot4(*reinterpret_cast<const float4*>(qrow + c), kv);
        da += dot4(*reinterpret_cast<const float4*>(a + c), kv);
        if (nb > 1) db += dot4(*reinterpret_cast<const float4*>(b + c), kv);
      }
    }
    if (!(valid && j <= qi)) return 0.f;
    return cached ? srow[j] : exp2f(ds * sc2 - m2);
  };

  // ---------------- right-hand side h = C^T g ----------------
  // U_j = w_j (g.v_j - g.out); h = (sum_j U_j k_j - (sum_j U_j) kbar) / omega
  // (any constant in place of g.out gives the same h: sum_j w_j (k_j - kbar) = 0)
  float usum = 0.f;
  for (int u = 0; u < YC; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  first(true);
  for (int kt = 0; kt < kend; kt += BKV) {
    next(kt, true);
    for (int u = 0; u < 2; ++u) {
      const int kc = ln + LPR * u;
      const int j = kt + kc;
      float dg = 0.f;
      for (int c = 0; c < D; c += 4)
        dg += dot4(*reinterpret_cast<const float4*>(grow + c),
                   *reinterpret_cast<const float4*>(sV + kc * LD + c));
      const float U = weight(kc, j) * (dg - gb);
      sW[row * LW + kc] = U;
      usum += U;
    }
    __syncthreads();
    tile_product(acc);
  }
  usum = group_sum<LPR>(usum);
  for (int u = 0; u < YC; ++u) acc[u] = slice_sum<CL, LPR>(acc[u]);
  float4 hv[YC], x[YC], r[YC];
  float rr = 0.f, kp = 0.f;
  for (int u = 0; u < YC; ++u) {
    const float4 a = acc[u];
    hv[u] = make_float4((a.x - usum * kb[u].x) * inv_om, (a.y - usum * kb[u].y) * inv_om,
                        (a.z - usum * kb[u].z) * inv_om, (a.w - usum * kb[u].w) * inv_om);
    x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    r[u] = hv[u];
    rr += dot4(r[u], r[u]);
    kp += dot4(kb[u], r[u]);
  }
  __syncthreads();
  if (sl == 0) {
    for (int u = 0; u < YC; ++u)
      *reinterpret_cast<float4*>(sP + row * LD + (cl + CL * u) * 4) = r[u];
  }
  rr = group_sum<CL>(rr);
  kp = group_sum<CL>(kp);
  const float r0 = sqrtf(rr);
  const float stop_at = P.cg_rel_tol * r0;
  bool active = valid && rr > 0.f && P.cg_max_iters > 0;
  int iters = 0;

  // ---------------- adjoint CG: Sigma_c y = h (the forward's loop) ----------------
  for (int it = 0; it < P.cg_max_iters; ++it) {
    if (tid == 0) sAny = 0;
    __syncthreads();
    if (active && ln == 0) sAny = 1;
    __syncthreads();
    if (!sAny) break;
    float us = 0.f;
    for (int u = 0; u < YC; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    first(false);
    for (int kt = 0; kt < kend; kt += BKV) {
      next(kt, false);
      for (int u = 0; u < 2; ++u) {
        const int kc = ln + LPR * u;
        const int j = kt + kc;
        float dt, unused;
        const float U = weight_dots(kc, j, 1, prow, dt, prow, unused) * (dt - kp);
        sW[row * LW + kc] = U;
        us += U;
      }
      __syncthreads();
      tile_product(acc);
    }
    us = group_sum<LPR>(us);
    for (int u = 0; u < YC; ++u) acc[u] = slice_sum<CL, LPR>(acc[u]);
    float pAp = 0.f;
    float4 Ap[YC], pv[YC];
    for (int u = 0; u < YC; ++u) {
      pv[u] = *reinterpret_cast<const float4*>(prow + (cl + CL * u) * 4);
      const float4 a = acc[u];
      Ap[u] = make_float4(a.x - us * kb[u].x + lam * pv[u].x, a.y - us * kb[u].y + lam * pv[u].y,
                          a.z - us * kb[u].z + lam * pv[u].z, a.w - us * kb[u].w + lam * pv[u].w);
      pAp += dot4(pv[u], Ap[u]);
    }
    pAp = group_sum<CL>(pAp);
    bool step = active && pAp > 0.f;
    if (active && !step) active = false;
    float rrn = 0.f;
    const float al = step ? rr / pAp : 0.f;
    for (int u = 0; u < YC; ++u) {
      if (step) {
        x[u] = fma4(al, pv[u], x[u]);
        r[u] = fma4(-al, Ap[u], r[u]);
      }
      rrn += dot4(r[u], r[u]);
    }
    rrn = group_sum<CL>(rrn);
    float kpn = 0.f;
    if (step) {
      ++iters;
      if (sqrtf(rrn) <= stop_at || rrn == 0.f) {
        active = false;
      } else {
        const float be = rrn / rr;
        for (int u = 0; u < YC; ++u) {
          pv[u] = fma4(be, pv[u], r[u]);
          // (every lane of the row has read p above: one wave holds the row)
          if (sl == 0) *reinterpret_cast<float4*>(sP + row * LD + (cl + CL * u) * 4) = pv[u];
          kpn += dot4(kb[u], pv[u]);
        }
      }
      rr = rrn;
    }
    kpn = group_sum<CL>(kpn);
    if (active) kp = kpn;
    __syncthreads();
  }
  if (valid && ln == 0) {
    if (P.adj_iters) P.adj_iters[orow / D] = iters;
    if (P.adj_resid) P.adj_resid[orow / D] = r0 > 0.f ? sqrtf(rr) / r0 : 0.f;
  }

  // ---------------- per-query constants ----------------
  __syncthreads();
  float4 rc[YC];
  float kbx = 0.f, kby = 0.f, kap = 0.f, yu = 0.f, yr = 0.f;
  for (int u = 0; u < YC; ++u) {
    const int c = (cl + CL * u) * 4;
    rc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) rc[u] = *reinterpret_cast<const float4*>(P.rho_c + orow + c);
    if (sl == 0) {
      *reinterpret_cast<float4*>(sP + row * LD + c) = rc[u];
      *reinterpret_cast<float4*>(sY + row * LD + c) = x[u];
    }
    kbx += dot4(kb[u], rc[u]);
    kby += dot4(kb[u], x[u]);
    kap += dot4(hv[u], rc[u]);
    yu += dot4(x[u], make_float4(kb[u].x - qv[u].x, kb[u].y - qv[u].y, kb[u].z - qv[u].z, kb[u].w - qv[u].w));
    yr += dot4(x[u], rc[u]);
  }
  kbx = group_sum<CL>(kbx);
  kby = group_sum<CL>(kby);
  kap = group_sum<CL>(kap);
  yu = group_sum<CL>(yu);
  yr = group_sum<CL>(yr);
  const float tau = valid ? kap * inv_om - yu : 0.f;
  const float msum = -lam * yr;
  const float gvbar = gb + kap;
  if (ln == 0) sOm[row] = inv_om;

  // ---------------- final sweep: dq, and dk, dv per key tile ----------------
  float rsum = 0.f;
  for (int u = 0; u < YC; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  first(true);
  for (int kt = 0; kt < kend; kt += BKV) {
    next(kt, true);
    for (int u = 0; u < 2; ++u) {
      const int kc = ln + LPR * u;
      const int j = kt + kc;
      float dr, dy, dg = 0.f;
      const float w = weight_dots(kc, j, 2, prow, dr, yrow, dy);
      for (int c = 0; c < D; c += 4)
        dg += dot4(*reinterpret_cast<const float4*>(grow + c),
                   *reinterpret_cast<const float4*>(sV + kc * LD + c));
      const bool vis = valid && j <= qi;
      const float A = 1.f - (dr - kbx);
      const float ev = (dg - gvbar) * inv_om - (dy - kby);
      const float sig = w * fmaf(A, ev, tau);
      rsum += sig;
      sW[row * LW + kc] = sig;
      sA[row * LW + kc] = cs * ((vis && j == bestj) ? sig - msum : sig);
      sB[row * LW + kc] = -w * A;
      sE[row * LW + kc] = -w * ev;
    }
    __syncthreads();
    tile_product(acc);
    // dk_j = sum_i [c dL/ds q_i - w A y_i - w e rho_c,i], dv_j = sum_i (w A / omega_i) g_i
    for (int e = tid; e < BKV * NC; e += VT) {
      const int kk = e / NC, c = (e % NC) * 4;
      const int j = kt + kk;
      if (j >= kend) continue;
      float4 dk = make_float4(0.f, 0.f, 0.f, 0.f), dv = dk;
      for (int i = 0; i < nq; ++i) {
        const float a1 = sA[i * LW + kk], a2 = sB[i * LW + kk], a3 = sE[i * LW + kk];
        dk = fma4(a1, *reinterpret_cast<const float4*>(sQ + i * LD + c), dk);
        dk = fma4(a2, *reinterpret_cast<const float4*>(sY + i * LD + c), dk);
        dk = fma4(a3, *reinterpret_cast<const float4*>(sP + i * LD + c), dk);
        dv = fma4(-a2 * sOm[i], *reinterpret_cast<const float4*>(sG + i * LD + c), dv);
      }
      float* pk = P.dk + base + static_cast<size_t>(j) * D + c;
      float* pvv = P.dv + base + static_cast<size_t>(j) * D + c;
      atomicAdd(pk + 0, dk.x); atomicAdd(pk + 1, dk.y); atomicAdd(pk + 2, dk.z); atomicAdd(pk + 3, dk.w);
      atomicAdd(pvv + 0, dv.x); atomicAdd(pvv + 1, dv.y); atomicAdd(pvv + 2, dv.z); atomicAdd(pvv + 3, dv.w);
    }
  }
  rsum = group_sum<LPR>(rsum);
  for (int u = 0; u < YC; ++u) acc[u] = slice_sum<CL, LPR>(acc[u]);
  if (!valid || sl != 0) return;
  // dq = c (sum_j dL/ds_j k_j - (sum_j dL/ds_j) k_j*) + omega y
  for (int u = 0; u < YC; ++u) {
    const int c = (cl + CL * u) * 4;
    const float4 ks = load4(K, static_cast<size_t>(bestj) * D + c);
    const float4 a = acc[u];
    const float4 o = make_float4(cs * (a.x - rsum * ks.x) + om * x[u].x, cs * (a.y - rsum * ks.y) + om * x[u].y,
                                 cs * (a.z - rsum * ks.z) + om * x[u].z, cs * (a.w - rsum * ks.w) + om * x[u].w);
    *reinterpret_cast<float4*>(P.dq + orow + c) = o;
  }
}

__global__ void zero_fill(float* __restrict__ a, float* __restrict__ b, size_t n4) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    reinterpret_cast<float4*>(a)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(b)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Lanes per query row for a launch: the fewest that still give every compute
// unit two workgroups; at most max_lpr.
template <int D>
hipError_t lanes_per_row(int n, int BH, int max_lpr, int* lpr) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long long fill = 2LL * cus;
  auto blocks = [&](int bq) { return static_cast<long long>((n + bq - 1) / bq) * BH; };
  *lpr = 8;
  while (*lpr < max_lpr && blocks(VT / *lpr) < fill) *lpr *= 2;
  return hipSuccess;
}

// Row stride of the weight cache (rows of n keys rounded up to the tile, plus
// LPR floats so that a wave's rows start on different banks), or 0 where the
// cache would take more than 64 KiB of dynamic LDS.
template <int D, int LPR>
int cache_stride(int n) {
  const long long ls = (static_cast<long long>(n) + 2 * LPR - 1) / (2 * LPR) * (2 * LPR) + LPR;
  return ls * Lanes<D, LPR>::VQ * 4 <= 65536 ? static_cast<int>(ls) : 0;
}

template <int D, typename Tin, int LPR>
hipError_t launch_bwd_lanes(const BwdParams& p, hipStream_t stream) {
  constexpr int BQ = Lanes<D, LPR>::VQ;
  const int nqb = (p.n + BQ - 1) / BQ;
  const long long blocks = static_cast<long long>(nqb) * p.BH;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t n4 = static_cast<size_t>(p.BH) * p.n * D / 4;
  hipLaunchKernelGGL(zero_fill, dim3(static_cast<unsigned>(std::min<size_t>((n4 + 255) / 256, 65536))), dim3(256), 0,
                     stream, p.dk, p.dv, n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_main_begin) {
    e = hipEventRecord(p.ev_main_begin, stream);
    if (e != hipSuccess) return e;
  }
  const int ls = cache_stride<D, LPR>(p.n);
  hipLaunchKernelGGL((lla_valu_bwd_kernel<D, Tin, LPR>), dim3(static_cast<unsigned>(blocks)), dim3(VT),
                     static_cast<unsigned>(ls) * BQ * 4u, stream, p, ls);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_main_end) return hipEventRecord(p.ev_main_end, stream);
  return hipSuccess;
}

template <int D, typename Tin>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  // one row per wave only for d <= 32: beyond, the two prefetched 128-key
  // tiles would not fit the registers the backward's state leaves
  int lpr = 8;
  const hipError_t e = lanes_per_row<D>(p.n, p.BH, D <= 32 ? 64 : 32, &lpr);
  if (e != hipSuccess) return e;
  if (lpr == 8) return launch_bwd_lanes<D, Tin, 8>(p, stream);
  if (lpr == 16) return launch_bwd_lanes<D, Tin, 16>(p, stream);
  if constexpr (D <= 32) {
    if (lpr == 64) return launch_bwd_lanes<D, Tin, 64>(p, stream);
  }
  return launch_bwd_lanes<D, Tin, 32>(p, stream);
}

template <typename Tin>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 16: return launch_bwd_d<16, Tin>(p, stream);
    case 32: return launch_bwd_d<32, Tin>(p, stream);
    case 64: return launch_bwd_d<64, Tin>(p, stream);
    case 128: return launch_bwd_d<128, Tin>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, typename Tin, int LPR>
hipError_t launch_lanes(const FwdParams& p, hipStream_t stream) {
  constexpr int BQ = Lanes<D, LPR>::VQ;
  const int nqb = (p.n + BQ - 1) / BQ;
  const long long blocks = static_cast<long long>(nqb) * p.BH;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.ev_main_begin) {
    const hipError_t e = hipEventRecord(p.ev_main_begin, stream);
    if (e != hipSuccess) return e;
  }
  const int ls = cache_stride<D, LPR>(p.n);
  hipLaunchKernelGGL((lla_valu_kernel<D, Tin, LPR>), dim3(static_cast<unsigned>(blocks)), dim3(VT),
                     static_cast<unsigned>(ls) * BQ * 4u, stream, p, ls);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_main_end) return hipEventRecord(p.ev_main_end, stream);
  return hipSuccess;
}

template <int D, typename Tin>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  // one row per wave (64 lanes) for d <= 64: at d = 128 the 128-key tiles
  // of K and V would not leave LDS for the weight cache
  int lpr = 8;
  const hipError_t e = lanes_per_row<D>(p.n, p.BH, D <= 64 ? 64 : 32, &lpr);
  if (e != hipSuccess) return e;
  if (lpr == 8) return launch_lanes<D, Tin, 8>(p, stream);
  if (lpr == 16) return launch_lanes<D, Tin, 16>(p, stream);
  if constexpr (D <= 64) {
    if (lpr == 64) return launch_lanes<D, Tin, 64>(p, stream);
  }
  return launch_lanes<D, Tin, 32>(p, stream);
}

template <typename Tin>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 16: return launch_d<16, Tin>(p, stream);
    case 32: return launch_d<32, Tin>(p, stream);
    case 64: return launch_d<64, Tin>(p, stream);
    case 128: return launch_d<128, Tin>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_valu(const FwdParams& p, hipStream_t stream) {
  if (p.dtype == LLA_DTYPE_F32) return launch_t<float>(p, stream);
  return launch_t<uint16_t>(p, stream);
}

hipError_t launch_valu_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.dtype == LLA_DTYPE_F32) return launch_bwd_t<float>(p, stream);
  return launch_bwd_t<uint16_t>(p, stream);
}

}  // namespace lla
