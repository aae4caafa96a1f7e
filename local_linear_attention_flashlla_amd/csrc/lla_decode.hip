// Decode-shaped LLA forward: one new query per (batch, head) against a cache
// of n keys and values, all of them visible (the last row of a causal forward
// whose query sits at position n - 1). Same estimator and CG policy as the
// blocked forward ("Local Linear Attention: reading notes", section 2.1,
// Eqs. (6)-(8); the CG of section 2.2 on the system centred at the weighted key
// mean, as described in include/lla.h).
//
// With a single query per head the matrix-free CG of the blocked forward has
// nothing to share a key fragment with: each iteration would re-read the whole
// cache for 2d multiply-adds per key on the vector ALU. Here the centred Gram
// matrix of the one query,
//     G = sum_j w_j (k_j - kbar)(k_j - kbar)^T        (d x d, independent of n),
// is formed once, as a dense product on the matrix cores split over the keys,
// and the CG iterations run on G + lambda I held in LDS: d^2 multiply-adds per
// iteration instead of 2 n d, and the cache is read three times in all (scores
// and moments, Gram, output) whatever the iteration count. In exact arithmetic
// the CG iterates are those of the matrix-free CG on the same system.
//
// Five kernels, the keys of each head split into S chunks of L:
//   dec_moments  (S x BH)  scores c q.k_j (kept, log2 units), chunk max, omega
//                          and mu~ partials;
//   dec_gram     (SG x BH) combines the partials into m, omega, kbar; the chunk's
//                          contribution to G = sum_j u_j u_j^T with
//                          u_j = sqrt(w_j) (k_j - kbar), on
//                          v_mfma_f32_32x32x16_f16, u carried as two fp16
//                          terms (hi + lo, ~22 bits): hi.hi + hi.lo + lo.hi;
//   dec_solve    (BH)      sums the chunk Grams, adds lambda I, runs CG on
//                          G rho_c = mu = omega (kbar - q);
//   dec_output   (S x BH)  a_j = w_j (1 - (k_j - kbar).rho_c): partial sums of
//                          a_j v_j and a_j;
//   dec_finish   (BH)      out = sum a_j v_j / sum a_j.
// No workgroup waits on another inside a kernel.

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "lla_internal.h"
#include "../../include/lla.h"

namespace lla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int DT = 256;        // threads per workgroup (four waves)
constexpr int GK = 32;         // keys per Gram tile
constexpr int GLD = GK + 8;    // LDS row stride (halfs) of the transposed Gram operands
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecParams {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  float* omega;
  float* rho;
  float* rowmax;
  int32_t* cg_iters;
  float* cg_resid;
  float* s;      // [BH][n] scores c q.k_j in log2 units
  float* p1;     // [BH][S][2 + d] chunk max, omega, mu~ (relative to the chunk max)
  float* gram;   // [BH][SG][d][d] chunk Grams
  float* st;     // [BH][2 d + 2] rho_c, kbar, m, omega
  float* p4;     // [BH][S][d + 1] sum a_j v_j, sum a_j
  int BH, n, S, L;     // key chunks of the score, moment and output kernels
  int SG, LG;          // key chunks of the Gram kernel (fewer: each writes d^2 floats)
  float lambda;
  int cg_max_iters;
  float cg_rel_tol;
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// the EPL = d / 64 consecutive elements of a row that lane `lane` owns
template <int D, typename T>
__device__ __forceinline__ void load_lane(const T* row, int lane, float (&x)[D / 64]) {
  #pragma unroll
  for (int e = 0; e < D / 64; ++e) x[e] = to_f(row[lane * (D / 64) + e]);
}

// Sum over the 64 lanes, the result in every lane, without the LDS crossbar:
// DPP quad permutations (partners l ^ 1, l ^ 2), row half-mirror and mirror
// (8- and 16-lane groups), then v_permlane16_swap and v_permlane32_swap,
// which exchange 16- and 32-lane halves.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_partner<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_partner<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_partner<0x141>(v);  // row_half_mirror
  v += dpp_partner<0x140>(v);  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Maximum over the 64 lanes, the same exchanges as wave_sum.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_partner<0xB1>(v));
  v = fmaxf(v, dpp_partner<0x4E>(v));
  v = fmaxf(v, dpp_partner<0x141>(v));
  v = fmaxf(v, dpp_partner<0x140>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Buffer resource over `bytes` bytes at `base` (reads past the end return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// The whole offset of a copy is the per-lane offset, which the buffer's range
// check covers: rows past the end of the cache read as zeros.
// The 32-key tiles of a chunk stream through four static LDS buffers: tile t
// (32 rows of the cache, contiguous in memory) is copied with
// buffer_load ... lds, 1 KiB per wave instruction, three steps before it is
// used, into buffer t % 4. Separate arrays keep every buffer choice static,
// so the compiler never waits on a copy it does not need.
template <int D, typename T>
struct Tiles {
  static constexpr int kBytes = GK * D * static_cast<int>(sizeof(T));
  static constexpr int kChunks = kBytes / 1024;
  static constexpr int kPerWave = kChunks / (DT / 64);  // copy instructions per wave and tile
  static_assert(kChunks % (DT / 64) == 0, "chunks must spread over the waves");
};
template <int D, typename T>
__device__ __forceinline__ void copy_tile(__amdgpu_buffer_rsrc_t r, uint32_t tile_off, T* buf, int wave,
                                          int lane) {
  #pragma unroll
  for (int u = 0; u < Tiles<D, T>::kPerWave; ++u) {
    const int ch = u * (DT / 64) + wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(reinterpret_cast<char*>(buf) + ch * 1024), 16,
        tile_off + ch * 1024 + lane * 16, 0, 0, 0);
  }
}
// Wait until at most N of this wave's copies are in flight and its LDS reads
// are done, then a barrier: every wave's older copies are then visible and no
// wave still reads a buffer that the next copy overwrites.
template <int N>
__device__ __forceinline__ void wait_copies_barrier() {
  static_assert(N == 2 || N == 4 || N == 6 || N == 8 || N == 10 || N == 12 || N == 16, "vmcnt below");
  if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int I> using IC = std::integral_constant<int, I>;

// m (log2 units), omega and kbar of head bh from the S <= 64 chunk partials:
// m = max_c m_c, omega = sum_c omega_c 2^(m_c - m), mu~ likewise, kbar = mu~ / omega.
// The first wave reads one chunk per lane (all loads in flight at once) and
// leaves the factors 2^(m_c - m) in sa[64]; threads t < D then sum their
// element of mu~ over the chunks, eight loads at a time. Writes kbar[t]
// (t < D), mo[0] = m, mo[1] = omega. Every thread of the block must call it.
template <int D>
__device__ __forceinline__ void combine_moments(const DecParams& P, int bh, float* kbar, float* mo, float* sa) {
  const float* base = P.p1 + static_cast<size_t>(bh) * P.S * (D + 2);
  const int t = threadIdx.x;
  if (t < 64) {
    const float mc = t < P.S ? base[t * (D + 2)] : -INFINITY;
    const float oc = t < P.S ? base[t * (D + 2) + 1] : 0.f;
    const float m = wave_max(mc);
    const float a = mc == -INFINITY ? 0.f : exp2f(mc - m);
    const float om = wave_sum(oc * a);
    sa[t] = a;
    if (t == 0) {
      mo[0] = m;
      mo[1] = om;
    }
  }
  __syncthreads();
  if (t < D) {
    float mu = 0.f;
    #pragma unroll 8
    for (int c = 0; c < P.S; ++c) mu += base[c * (D + 2) + 2 + t] * sa[c];
    kbar[t] = mu / mo[1];
  }
}

// --------------------------- scores and moments ----------------------------
template <int D, typename T>
__global__ __launch_bounds__(DT) void dec_moments(DecParams P) {
  constexpr int KPW = GK / (DT / 64);  // keys of a tile per wave
  constexpr int LPK = 64 / KPW;        // lanes per key
  constexpr int DPL = D / LPK;         // dimensions of its key that a lane holds
  static_assert(LPK == 8, "a key's score is an 8-lane butterfly");
  __shared__ __align__(16) T b0[GK * D], b1[GK * D], b2[GK * D], b3[GK * D];
  __shared__ float sm[DT / 64], som[DT / 64];
  __shared__ float smu[DT / 64][D];
  auto BUF = [&](auto I) __attribute__((always_inline)) -> T* {
    constexpr int i = decltype(I)::value % 4;
    if constexpr (i == 0) return b0;
    else if constexpr (i == 1) return b1;
    else if constexpr (i == 2) return b2;
    else return b3;
  };
  const int sp = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // lane = LPK * slot + part: key `slot` of the wave's KPW keys of a tile,
  // dimensions [DPL part, DPL (part + 1)) of it
  const int slot = lane / LPK, part = lane % LPK;
  const int c0 = sp * P.L, c1 = min(P.n, c0 + P.L);
  const int ntl = (c1 - c0 + GK - 1) / GK;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(static_cast<const T*>(P.k) + static_cast<size_t>(bh) * P.n * D,
                                              static_cast<uint32_t>(static_cast<size_t>(P.n) * D * sizeof(T)));
  auto toff = [&](int t) __attribute__((always_inline)) {
    return static_cast<uint32_t>((c0 + min(t, ntl - 1) * GK) * D * static_cast<int>(sizeof(T)));
  };
  float qd[DPL];
  {
    const T* qrow = static_cast<const T*>(P.q) + static_cast<size_t>(bh) * D + part * DPL;
    #pragma unroll
    for (int e = 0; e < DPL; ++e) qd[e] = to_f(qrow[e]);
  }
  const float cs = kLog2e / sqrtf(static_cast<float>(D));
  // running max (the same in every lane), this lane's share of omega (lanes
  // with part 0 count their key) and of mu~ (its key slot's keys, its dims)
  float m = -INFINITY, om = 0.f, mu[DPL];
  #pragma unroll
  for (int e = 0; e < DPL; ++e) mu[e] = 0.f;
  copy_tile<D>(kr, toff(0), b0, wave, lane);
  copy_tile<D>(kr, toff(1), b1, wave, lane);
  copy_tile<D>(kr, toff(2), b2, wave, lane);
  // step t: tile t has landed; copy tile t + 3 (clamped: every step issues the
  // same number of copies); this wave's KPW keys of tile t, one per 8 lanes
  auto step = [&](auto JM, int t) __attribute__((always_inline)) {
    wait_copies_barrier<2 * Tiles<D, T>::kPerWave>();
    copy_tile<D>(kr, toff(t + 3), BUF(IC<decltype(JM)::value + 3>{}), wave, lane);
    if (t >= ntl) return;  // block-uniform
    const T* row = BUF(JM) + (KPW * wave + slot) * D + part * DPL;
    float kd[DPL];
    float s = 0.f;
    #pragma unroll
    for (int e = 0; e < DPL; ++e) {
      kd[e] = to_f(row[e]);
      s += qd[e] * kd[e];
    }
    // the key's 8 lanes: a butterfly of commutative adds, so all 8 hold the
    // same sum
    s += dpp_partner<0xB1>(s);   // quad_perm [1, 0, 3, 2]
    s += dpp_partner<0x4E>(s);   // quad_perm [2, 3, 0, 1]
    s += dpp_partner<0x141>(s);  // row_half_mirror
    const int j = c0 + t * GK + KPW * wave + slot;
    const bool in = j < c1;
    const float sj = in ? s * cs : -INFINITY;
    if (in && part == 0) P.s[static_cast<size_t>(bh) * P.n + j] = sj;
    const float tmax = wave_max(sj);
    if (tmax > m) {  // wave-uniform; exp2(-inf) = 0 on the first keys
      const float a = exp2f(m - tmax);
      om *= a;
      #pragma unroll
      for (int e = 0; e < DPL; ++e) mu[e] *= a;
      m = tmax;
    }
    const float w = in ? exp2f(sj - m) : 0.f;  // (m is -inf while no key has been seen)
    if (part == 0) om += w;
    #pragma unroll
    for (int e = 0; e < DPL; ++e) mu[e] += w * kd[e];
  };
  for (int t0 = 0; t0 < ntl; t0 += 4) {
    step(IC<0>{}, t0);
    step(IC<1>{}, t0 + 1);
    step(IC<2>{}, t0 + 2);
    step(IC<3>{}, t0 + 3);
  }
  // the wave's totals: omega over all lanes, mu~ over the KPW key slots
  // (lanes part, part + 8, ..., part + 56)
  om = wave_sum(om);
  #pragma unroll
  for (int e = 0; e < DPL; ++e) {
    mu[e] += __shfl_xor(mu[e], 8);
    mu[e] += __shfl_xor(mu[e], 16);
    mu[e] += __shfl_xor(mu[e], 32);
  }
  if (lane == 0) {
    sm[wave] = m;
    som[wave] = om;
  }
  if (slot == 0) {
    #pragma unroll
    for (int e = 0; e < DPL; ++e) smu[wave][part * DPL + e] = mu[e];
  }
  __syncthreads();  // (also: no tile copy is still in flight past this point)
  const int t = threadIdx.x;
  if (t < D) {
    float mc = -INFINITY;
    #pragma unroll
    for (int w = 0; w < DT / 64; ++w) mc = fmaxf(mc, sm[w]);
    float o = 0.f, u = 0.f;
    #pragma unroll
    for (int w = 0; w < DT / 64; ++w) {
      if (sm[w] == -INFINITY) continue;
      const float a = exp2f(sm[w] - mc);
      o += som[w] * a;
      u += smu[w][t] * a;
    }
    float* dst = P.p1 + (static_cast<size_t>(bh) * P.S + sp) * (D + 2);
    if (t == 0) {
      dst[0] = mc;
      dst[1] = o;
    }
    dst[2 + t] = u;
  }
}

// ------------------------------ chunk Gram ---------------------------------
template <int D, typename T>
__global__ __launch_bounds__(DT) void dec_gram(DecParams P) {
  constexpr int NB = D / 32;                     // 32-row blocks of G
  constexpr int NT = NB * (NB + 1) / 2;          // blocks on or above the diagonal (G is symmetric)
  constexpr int TPW = (NT + DT / 64 - 1) / (DT / 64);  // output tiles per wave (the last may be empty)
  // upper-triangle tile t -> block row I and column J >= I
  auto tile_of = [](int t, int& I, int& J) __attribute__((always_inline)) {
    I = 0;
    #pragma unroll
    for (int r = 0; r < NB; ++r)
      if (t >= NB - I) {
        t -= NB - I;
        ++I;
      }
    J = I + t;
  };
  constexpr int IPT = D * (GK / 8) / DT;    // staging items (one d, 8 keys) per thread
  static_assert(IPT * DT == D * (GK / 8), "items must spread evenly");
  __shared__ __align__(16) T r0[GK * D], r1[GK * D], r2[GK * D], r3[GK * D];
  __shared__ __align__(16) _Float16 uHi[D * GLD], uLo[D * GLD];
  __shared__ float skb[D];
  __shared__ __align__(16) float sw[2][GK];
  __shared__ float smo[2], sca[64];
  auto RB = [&](auto I) __attribute__((always_inline)) -> T* {
    constexpr int i = decltype(I)::value % 4;
    if constexpr (i == 0) return r0;
    else if constexpr (i == 1) return r1;
    else if constexpr (i == 2) return r2;
    else return r3;
  };
  const int sp = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = sp * P.LG, c1 = min(P.n, c0 + P.LG);
  const int ntl = (c1 - c0 + GK - 1) / GK;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(static_cast<const T*>(P.k) + static_cast<size_t>(bh) * P.n * D,
                                              static_cast<uint32_t>(static_cast<size_t>(P.n) * D * sizeof(T)));
  auto toff = [&](int t) __attribute__((always_inline)) {
    return static_cast<uint32_t>((c0 + min(t, ntl - 1) * GK) * D * static_cast<int>(sizeof(T)));
  };
  copy_tile<D>(kr, toff(0), r0, wave, lane);
  copy_tile<D>(kr, toff(1), r1, wave, lane);
  copy_tile<D>(kr, toff(2), r2, wave, lane);
  combine_moments<D>(P, bh, skb, smo, sca);
  __syncthreads();
  const float m = smo[0];
  const float* S = P.s + static_cast<size_t>(bh) * P.n;
  // scores of key tid of tiles t .. t + 3 in a ring (threads tid < GK); the
  // weights of tile t + 1 are written to LDS during step t
  float sR[4] = {0.f, 0.f, 0.f, 0.f};
  auto load_s = [&](int t) __attribute__((always_inline)) {
    const int j = c0 + t * GK + tid;
    return (tid < GK && j < c1) ? S[j] : -INFINITY;
  };
  sR[0] = load_s(0);
  sR[1] = load_s(1);
  sR[2] = load_s(2);
  // sw holds sqrt(w) = 2^((s - m) / 2): the chunk Gram is sum_j u_j u_j^T with
  // u_j = sqrt(w_j) (k_j - kbar); keys past the chunk: 0
  if (tid < GK) sw[0][tid] = exp2f(0.5f * (sR[0] - m));
  floatx16 acc[TPW];
  #pragma unroll
  for (int u = 0; u < TPW; ++u)
    #pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
  auto step = [&](auto JM, int t) __attribute__((always_inline)) {
    constexpr int jm = decltype(JM)::value;
    // raw tile t has landed; every wave is done with the operands of tile t - 1
    wait_copies_barrier<2 * Tiles<D, T>::kPerWave>();
    copy_tile<D>(kr, toff(t + 3), RB(IC<jm + 3>{}), wave, lane);
    if (t >= ntl) return;  // block-uniform
    if (tid < GK) sw[(jm + 1) & 1][tid] = exp2f(0.5f * (sR[(jm + 1) % 4] - m));
    sR[(jm + 3) % 4] = load_s(t + 3);
    // transposed operand: row d holds the tile's keys of u = sqrt(w) (k - kbar)
    // as fp16 hi + lo
    const T* raw = RB(JM);
    const float* w = sw[jm & 1];
    #pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + DT * i, d = it % D, kg = it / D;
      const float kbd = skb[d];
      // every tile buffer holds GK copied rows (past the chunk: the next
      // chunk's keys, or zeros past the cache), so every read is in bounds;
      // keys past the chunk have sqrt(w) = 0, so their (finite) k - kbar
      // gives u = 0 and needs no mask
      const float4 w0 = *reinterpret_cast<const float4*>(w + 8 * kg);
      const float4 w1 = *reinterpret_cast<const float4*>(w + 8 * kg + 4);
      const float we[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      half8 uh, ul;
      #pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 8 * kg + e;
        const float u = we[e] * (to_f(raw[kk * D + d]) - kbd);
        uh[e] = static_cast<_Float16>(u);
        ul[e] = static_cast<_Float16>(u - static_cast<float>(uh[e]));
      }
      *reinterpret_cast<half8*>(uHi + d * GLD + 8 * kg) = uh;
      *reinterpret_cast<half8*>(uLo + d * GLD + 8 * kg) = ul;
    }
    __syncthreads();
    #pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks)
      #pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int ti = wave + (DT / 64) * u;
        if (ti >= NT) continue;  // wave-uniform
        int I, J;
        tile_of(ti, I, J);
        const int ao = (32 * I + ql) * GLD + 16 * ks + 8 * g;
        const int bo = (32 * J + ql) * GLD + 16 * ks + 8 * g;
        const half8 ah = *reinterpret_cast<const half8*>(uHi + ao);
        const half8 al = *reinterpret_cast<const half8*>(uLo + ao);
        const half8 bhv = *reinterpret_cast<const half8*>(uHi + bo);
        const half8 blv = *reinterpret_cast<const half8*>(uLo + bo);
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bhv, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, blv, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bhv, acc[u], 0, 0, 0);
      }
  };
  for (int t0 = 0; t0 < ntl; t0 += 4) {
    step(IC<0>{}, t0);
    step(IC<1>{}, t0 + 1);
    step(IC<2>{}, t0 + 2);
    step(IC<3>{}, t0 + 3);
  }
  __syncthreads();  // no tile copy may still be in flight when the kernel ends
  // accumulator register r of lane (ql, g) holds row 8 (r / 4) + 4 g + r % 4,
  // column ql of its 32 x 32 tile
  float* G = P.gram + (static_cast<size_t>(bh) * P.SG + sp) * D * D;
  #pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int ti = wave + (DT / 64) * u;
    if (ti >= NT) continue;  // wave-uniform
    int I, J;
    tile_of(ti, I, J);
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * I + 8 * (r >> 2) + 4 * g + (r & 3);
      G[i * D + 32 * J + ql] = acc[u][r];
      if (I != J) G[(32 * J + ql) * D + i] = acc[u][r];  // the mirror block
    }
  }
}

// ---------------------------------- solve ----------------------------------
// Block-wide sum of one value per thread of the first D threads (the others
// pass 0); every thread gets the total.
template <int D>
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();  // red may still be read by the previous call
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  #pragma unroll
  for (int w = 0; w < DT / 64; ++w) s += red[w];
  return s;
}

template <int D, typename T>
__global__ __launch_bounds__(DT) void dec_solve(DecParams P) {
  constexpr int LG = D + 1;          // row stride of G in LDS
  constexpr int NP = DT / D;         // column parts of the matrix-vector product
  __shared__ float sG[D * LG];
  __shared__ float skb[D], sp_[D], spart[NP][D];
  __shared__ float smo[2], red[DT / 64], sca[64];
  const int bh = blockIdx.x, t = threadIdx.x;
  combine_moments<D>(P, bh, skb, smo, sca);
  // G + lambda I from the chunk Grams: each thread sums its NG float4s of G
  // over the chunks in order, all NG loads of a chunk in flight together
  constexpr int NG = D * D / 4 / DT;
  static_assert(NG * 4 * DT == D * D, "G must spread evenly over the threads");
  const float4* Gc = reinterpret_cast<const float4*>(P.gram + static_cast<size_t>(bh) * P.SG * D * D);
  float4 ga[NG];
  #pragma unroll
  for (int u = 0; u < NG; ++u) ga[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  // two chunks per round trip (2 NG loads in flight), added in chunk order
  int c = 0;
  for (; c + 1 < P.SG; c += 2) {
    const float4* g0 = Gc + static_cast<size_t>(c) * (D * D / 4);
    const float4* g1 = g0 + D * D / 4;
    float4 a0[NG], a1[NG];
    #pragma unroll
    for (int u = 0; u < NG; ++u) {
      a0[u] = g0[t + DT * u];
      a1[u] = g1[t + DT * u];
    }
    #pragma unroll
    for (int u = 0; u < NG; ++u) {
      ga[u].x += a0[u].x; ga[u].y += a0[u].y; ga[u].z += a0[u].z; ga[u].w += a0[u].w;
      ga[u].x += a1[u].x; ga[u].y += a1[u].y; ga[u].z += a1[u].z; ga[u].w += a1[u].w;
    }
  }
  if (c < P.SG) {
    const float4* gc = Gc + static_cast<size_t>(c) * (D * D / 4);
    #pragma unroll
    for (int u = 0; u < NG; ++u) {
      const float4 g = gc[t + DT * u];
      ga[u].x += g.x; ga[u].y += g.y; ga[u].z += g.z; ga[u].w += g.w;
    }
  }
  #pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int idx = 4 * (t + DT * u), i = idx / D, j = idx % D;
    const float e[4] = {ga[u].x, ga[u].y, ga[u].z, ga[u].w};
    #pragma unroll
    for (int q = 0; q < 4; ++q) sG[i * LG + j + q] = e[q] + (i == j + q ? P.lambda : 0.f);
  }
  __syncthreads();
  const float m = smo[0], om = smo[1];
  // CG on (G + lambda I) x = mu = omega (kbar - q): thread t < D owns element t
  const bool own = t < D;
  float qv = 0.f, kb = 0.f, x = 0.f, r = 0.f, p = 0.f;
  if (own) {
    qv = to_f(static_cast<const T*>(P.q)[static_cast<size_t>(bh) * D + t]);
    kb = skb[t];
    r = om * (kb - qv);
    p = r;
  }
  float rr = block_sum<D>(own ? r * r : 0.f, red);
  const float r0 = sqrtf(rr);
  const float thr = P.cg_rel_tol * r0;
  bool active = rr > 0.f && P.cg_max_iters > 0;
  int iters = 0;
  const int row = t % D, part = t / D;
  for (int it = 0; it < P.cg_max_iters && active; ++it) {  // `active` is block-uniform
    if (own) sp_[t] = p;
    __syncthreads();
    float ap = 0.f;
    #pragma unroll 8
    for (int c = part * (D / NP); c < (part + 1) * (D / NP); ++c) ap += sG[row * LG + c] * sp_[c];
    spart[part][row] = ap;
    __syncthreads();
    float Ap = 0.f;
    if (own) {
      #pragma unroll
      for (int h = 0; h < NP; ++h) Ap += spart[h][t];
    }
    const float pAp = block_sum<D>(own ? p * Ap : 0.f, red);
    if (!(pAp > 0.f)) break;  // breakdown: keep the iterate
    const float al = rr / pAp;
    x += al * p;
    r -= al * Ap;
    const float rrn = block_sum<D>(own ? r * r : 0.f, red);
    ++iters;
    if (sqrtf(rrn) <= thr || rrn == 0.f) {
      rr = rrn;
      break;
    }
    p = r + (rrn / rr) * p;
    rr = rrn;
  }
  // state for the output scan; the pages' rho_i = rho_c / (1 + (kbar - q).rho_c)
  const float kq = block_sum<D>(own ? (kb - qv) * x : 0.f, red);
  if (own) {
    float* st = P.st + static_cast<size_t>(bh) * (2 * D + 2);
    st[t] = x;
    st[D + t] = kb;
    if (t == 0) {
      st[2 * D] = m;
      st[2 * D + 1] = om;
    }
    if (P.rho) P.rho[static_cast<size_t>(bh) * D + t] = x / (1.f + kq);
  }
  if (t == 0) {
    if (P.omega) P.omega[bh] = om;
    if (P.rowmax) P.rowmax[bh] = m * kLn2;
    if (P.cg_iters) P.cg_iters[bh] = iters;
    if (P.cg_resid) P.cg_resid[bh] = r0 > 0.f ? sqrtf(rr) / r0 : 0.f;
  }
}

// ---------------------------------- output ---------------------------------
template <int D, typename T>
__global__ __launch_bounds__(DT) void dec_output(DecParams P) {
  constexpr int KPW = GK / (DT / 64);
  __shared__ __align__(16) T k0[GK * D], k1[GK * D], k2[GK * D], k3[GK * D];
  __shared__ __align__(16) T v0[GK * D], v1[GK * D], v2[GK * D], v3[GK * D];
  __shared__ float sden[DT / 64];
  __shared__ float so[DT / 64][D];
  auto KB = [&](auto I) __attribute__((always_inline)) -> T* {
    constexpr int i = decltype(I)::value % 4;
    if constexpr (i == 0) return k0;
    else if constexpr (i == 1) return k1;
    else if constexpr (i == 2) return k2;
    else return k3;
  };
  auto VB = [&](auto I) __attribute__((always_inline)) -> T* {
    constexpr int i = decltype(I)::value % 4;
    if constexpr (i == 0) return v0;
    else if constexpr (i == 1) return v1;
    else if constexpr (i == 2) return v2;
    else return v3;
  };
  const int sp = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = sp * P.L, c1 = min(P.n, c0 + P.L);
  const int ntl = (c1 - c0 + GK - 1) / GK;
  const uint32_t head_bytes = static_cast<uint32_t>(static_cast<size_t>(P.n) * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t kr =
      make_rsrc(static_cast<const T*>(P.k) + static_cast<size_t>(bh) * P.n * D, head_bytes);
  const __amdgpu_buffer_rsrc_t vr =
      make_rsrc(static_cast<const T*>(P.v) + static_cast<size_t>(bh) * P.n * D, head_bytes);
  auto toff = [&](int t) __attribute__((always_inline)) {
    return static_cast<uint32_t>((c0 + min(t, ntl - 1) * GK) * D * static_cast<int>(sizeof(T)));
  };
  // lane = LPK * slot + part: key `slot` of the wave's KPW keys of a tile,
  // dimensions [DPL part, DPL (part + 1)) of it
  constexpr int LPK = 64 / KPW, DPL = D / LPK;
  static_assert(LPK == 8, "a key's dot product is an 8-lane butterfly");
  const int slot = lane / LPK, part = lane % LPK;
  const float* st = P.st + static_cast<size_t>(bh) * (2 * D + 2);
  float xr[DPL], kr_dot = 0.f;
  #pragma unroll
  for (int e = 0; e < DPL; ++e) {
    xr[e] = st[part * DPL + e];
    kr_dot += st[D + part * DPL + e] * xr[e];
  }
  // kbar . rho_c over the 8 parts (every key slot holds the same copy)
  kr_dot += dpp_partner<0xB1>(kr_dot);
  kr_dot += dpp_partner<0x4E>(kr_dot);
  kr_dot += dpp_partner<0x141>(kr_dot);
  const float m = st[2 * D];
  const float* S = P.s + static_cast<size_t>(bh) * P.n;
  float o[DPL], den = 0.f;
  #pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  // the score of this lane's key, loaded two steps ahead into a ring of four
  float sreg[4];
  auto load_s = [&](int t) __attribute__((always_inline)) {
    const int j = c0 + t * GK + KPW * wave + slot;
    return j < c1 ? S[j] : -INFINITY;  // past the chunk: weight 0
  };
  sreg[0] = load_s(0);
  sreg[1] = load_s(1);
  copy_tile<D>(kr, toff(0), k0, wave, lane);
  copy_tile<D>(vr, toff(0), v0, wave, lane);
  copy_tile<D>(kr, toff(1), k1, wave, lane);
  copy_tile<D>(vr, toff(1), v1, wave, lane);
  copy_tile<D>(kr, toff(2), k2, wave, lane);
  copy_tile<D>(vr, toff(2), v2, wave, lane);
  auto step = [&](auto JM, int t) __attribute__((always_inline)) {
    wait_copies_barrier<4 * Tiles<D, T>::kPerWave>();
    copy_tile<D>(kr, toff(t + 3), KB(IC<decltype(JM)::value + 3>{}), wave, lane);
    copy_tile<D>(vr, toff(t + 3), VB(IC<decltype(JM)::value + 3>{}), wave, lane);
    if (t >= ntl) return;  // block-uniform
    constexpr int jm = decltype(JM)::value;
    sreg[(jm + 2) % 4] = load_s(t + 2);
    const int ro = (KPW * wave + slot) * D + part * DPL;
    const T* kb = KB(JM) + ro;
    const T* vb = VB(JM) + ro;
    float vd[DPL], dot = 0.f;
    #pragma unroll
    for (int e = 0; e < DPL; ++e) {
      dot += to_f(kb[e]) * xr[e];
      vd[e] = to_f(vb[e]);
    }
    dot += dpp_partner<0xB1>(dot);   // quad_perm [1, 0, 3, 2]
    dot += dpp_partner<0x4E>(dot);   // quad_perm [2, 3, 0, 1]
    dot += dpp_partner<0x141>(dot);  // row_half_mirror
    const float a = exp2f(sreg[jm] - m) * (1.f - (dot - kr_dot));
    if (part == 0) den += a;
    #pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] += a * vd[e];
  };
  for (int t0 = 0; t0 < ntl; t0 += 4) {
    step(IC<0>{}, t0);
    step(IC<1>{}, t0 + 1);
    step(IC<2>{}, t0 + 2);
    step(IC<3>{}, t0 + 3);
  }
  // the wave's totals: den over all lanes, o over the KPW key slots
  den = wave_sum(den);
  #pragma unroll
  for (int e = 0; e < DPL; ++e) {
    o[e] += __shfl_xor(o[e], 8);
    o[e] += __shfl_xor(o[e], 16);
    o[e] += __shfl_xor(o[e], 32);
  }
  if (lane == 0) sden[wave] = den;
  if (slot == 0) {
    #pragma unroll
    for (int e = 0; e < DPL; ++e) so[wave][part * DPL + e] = o[e];
  }
  __syncthreads();  // (also: no tile copy is still in flight past this point)
  const int t = threadIdx.x;
  if (t <= D) {
    float a = 0.f;
    #pragma unroll
    for (int w = 0; w < DT / 64; ++w) a += t < D ? so[w][t] : sden[w];
    P.p4[(static_cast<size_t>(bh) * P.S + sp) * (D + 1) + t] = a;
  }
}

template <int D>
__global__ __launch_bounds__(DT) void dec_finish(DecParams P) {
  const int bh = blockIdx.x, t = threadIdx.x;
  if (t >= D) return;
  const float* p4 = P.p4 + static_cast<size_t>(bh) * P.S * (D + 1);
  float o = 0.f, den = 0.f;
  #pragma unroll 8
  for (int c = 0; c < P.S; ++c) {
    o += p4[c * (D + 1) + t];
    den += p4[c * (D + 1) + D];
  }
  P.out[static_cast<size_t>(bh) * D + t] = o / den;
}

// ============================ single pass (bf16) ============================
// For bf16 caches the moments, the Gram matrix and the cross moment all come
// from one read of K and V. With weights w_j = 2^(s_j - m) against the
// chunk's own max, a chunk of keys yields
//     omega_c, sum w k, sum w v, G_c = sum_j (w_j k_j) k_j^T, C_c = sum_j (w_j v_j) k_j^T,
// and the head's system follows from the chunk sums (each scaled by
// 2^(m_c - m)) by the parallel-axis identity:
//     Sigma_c = G - omega kbar kbar^T + lambda I,  mu = omega (kbar - q),
// and, since sum_j w_j (k_j - kbar) = 0 makes sum_j a_j = omega,
//     out = (sum w v - C rho_c + (sum w v)(kbar . rho_c)) / omega
// (the covariance form of the output: the Parallax summary's identity, here
// with the expansion point kbar). The products run on
// v_mfma_f32_32x32x16_bf16: a raw bf16 key is exact as an operand and bf16
// keeps fp32's exponent range, so no scale is needed; w k and w v are carried
// as two bf16 terms (hi + lo, about 16 bits), which puts the decode within
// about 1e-5 of the float64 CG on the test recipes.
//
//   dec1_chunk (S x BH)  one pass over a chunk of L keys: partials m_c, omega_c,
//                        sum w k, sum w v, G_c, C_c;
//   dec1_combine         (S > 1 only) the partials of a head summed into one;
//   dec1_solve (BH)      CG on Sigma_c in fp32, the output above and the
//                        optional outputs.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct Dec1Params {
  const uint16_t* q;  // [BH][D] bf16
  const uint16_t* k;  // [BH][n][D] bf16
  const uint16_t* v;
  float* out;
  float* omega;
  float* rho;
  float* rowmax;
  int32_t* cg_iters;
  float* cg_resid;
  float* part;        // [BH][S][PSZ] chunk partials (layout below)
  float* comb;        // [BH][PSZ] the chunk partials of a head combined (S > 1)
  int BH, n, S, L;    // S chunks of L keys (L a multiple of 32)
  float lambda;
  int cg_max_iters;
  float cg_rel_tol;
};

// One chunk's partials, PSZ floats: [0] m_c (the chunk's max score, log2
// units), [1] omega_c, [2, 3] unused, then sum w k (D), sum w v (D), G_c (D x D,
// row-major), C_c (D x D, row i = value dimension); weights against m_c.
template <int D>
struct Dec1Shape {
  static constexpr int NB = D / 32;                  // 32-row blocks of G and of C
  static constexpr int NW = 2 * NB;                  // waves: NB for G's rows, NB for C's
  static constexpr int NT = 64 * NW;
  static constexpr int KLD = GK + 8;                 // row stride (bf16) of the transposed key tile
  static constexpr int PSZ = 4 + 2 * D + 2 * D * D;
  static_assert(GK * D * 2 / 1024 == NW, "each wave copies one KiB of K and one of V per tile");
};

// A chunk's weights are taken against the max of its first tile and scaled
// once, at the end, to the chunk's exact max. A weight may exceed 1 there by
// up to this many binades (bf16 operands and fp32 sums hold it); should a
// later tile pass the first one's max by more, the chunk is formed a second
// time against its exact max, which the first pass has found (a restart, not
// a rescale of the accumulators mid-stream).
constexpr float kRaise = 40.f;

// Raw tiles in flight: a ring of NR tiles of K and of V, copied NR - 1 tiles
// ahead (even, so that a tile's parity follows its slot)
constexpr int NR = 6;
static_assert(NR % 2 == 0, "tile parity must follow the ring slot");

template <int D>
__device__ __forceinline__ void copy_kib(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t* buf, int wave,
                                         int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(reinterpret_cast<char*>(buf) + wave * 1024), 16,
      off + wave * 1024 + lane * 16, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(Dec1Shape<D>::NT) void dec1_chunk(Dec1Params P) {
  using SH = Dec1Shape<D>;
  constexpr int NB = SH::NB, KLD = SH::KLD, NKS = D / 32;
  // raw tiles (32 keys of K and of V, bf16 as stored) in a ring of six,
  // copied five tiles ahead (the latency of a loaded HBM is long); the
  // transposed key tile (B operand of every product; two halves of D / 2
  // rows) and the tile's weights double-buffered. The ring slots are the
  // largest LDS objects, so they take the lowest 96 KiB: every LDS address
  // the copies write stays below that.
  __shared__ __align__(16) uint16_t k0[GK * D], k1[GK * D], k2[GK * D], k3[GK * D], k4[GK * D], k5[GK * D];
  __shared__ __align__(16) uint16_t v0[GK * D], v1[GK * D], v2[GK * D], v3[GK * D], v4[GK * D], v5[GK * D];
  __shared__ __align__(16) uint16_t kt0a[D / 2 * KLD], kt0b[D / 2 * KLD], kt1a[D / 2 * KLD], kt1b[D / 2 * KLD];
  __shared__ __align__(16) float sw0[GK], sw1[GK];
  __shared__ float sred[SH::NW][3], sm0[SH::NW];
  static_assert(GK * D > D / 2 * KLD, "the ring slots must be the largest LDS objects");
  auto KB = [&](auto I) __attribute__((always_inline)) -> uint16_t* {
    constexpr int i = decltype(I)::value % NR;
    if constexpr (i == 0) return k0;
    else if constexpr (i == 1) return k1;
    else if constexpr (i == 2) return k2;
    else if constexpr (i == 3) return k3;
    else if constexpr (i == 4) return k4;
    else return k5;
  };
  auto VB = [&](auto I) __attribute__((always_inline)) -> uint16_t* {
    constexpr int i = decltype(I)::value % NR;
    if constexpr (i == 0) return v0;
    else if constexpr (i == 1) return v1;
    else if constexpr (i == 2) return v2;
    else if constexpr (i == 3) return v3;
    else if constexpr (i == 4) return v4;
    else return v5;
  };
  // rows [0, D / 2) and [D / 2, D) of the transposed key tile of parity I
  auto KT = [&](auto I, auto H) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(I)::value % 2 == 0) return decltype(H)::value ? kt0b : kt0a;
    else return decltype(H)::value ? kt1b : kt1a;
  };
  auto SW = [&](auto I) __attribute__((always_inline)) -> float* {
    if constexpr (decltype(I)::value % 2 == 0) return sw0;
    else return sw1;
  };
  const int sp = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool kwave = wave < NB;             // rows of G (else rows of C)
  const int brow = kwave ? wave : wave - NB;
  const int c0 = sp * P.L, c1 = min(P.n, c0 + P.L);
  const int ntl = (c1 - c0 + GK - 1) / GK;  // >= 1: every chunk holds keys
  // the sweep runs a multiple of NR steps (one loop exit, no branch around
  // the products): tiles past the chunk are masked, weight 0, and add nothing
  const int ntlr = (ntl + NR - 1) / NR * NR;
  const size_t hoff = static_cast<size_t>(bh) * P.n * D;
  const uint32_t hbytes = static_cast<uint32_t>(static_cast<size_t>(P.n) * D * sizeof(uint16_t));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(P.k + hoff, hbytes), vr = make_rsrc(P.v + hoff, hbytes);
  // tiles past the chunk are clamped copies of its last tile (finite, masked)
  auto copy = [&](auto I, int t) __attribute__((always_inline)) {
    const uint32_t off = static_cast<uint32_t>((c0 + min(t, ntl - 1) * GK) * D * sizeof(uint16_t));
    copy_kib<D>(kr, off, KB(I), wave, lane);
    copy_kib<D>(vr, off, VB(I), wave, lane);
  };

  // ---- scores: every wave scores KPW = 32 / NW keys of the next tile every
  // step (no branch, so the compiler interleaves them with the staging), on
  // v_mfma_f32_16x16x32_bf16: A = the raw key rows (rows l16 repeat the
  // wave's keys), B = q in every column; lane (l16, g4) gets row 4 g4 + e,
  // key KPW wave + (4 g4 + e) % KPW
  constexpr int KPW = GK / SH::NW;  // 4 (d = 128) or 8 (d = 64)
  static_assert(KPW == 4 || KPW == 8, "keys per wave");
  const int l16 = lane & 15, g4 = lane >> 4;
  bf16x8 qf[NKS];
  {
    const uint16_t* qh = P.q + static_cast<size_t>(bh) * D;
    #pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qh + 32 * ks + 8 * g4));
  }
  const float cs = kLog2e / sqrtf(static_cast<float>(D));
  // the reference (tile 0's max, the same in every wave); this wave's exact
  // max and sum of weights over its keys, and `over`: one of its keys passed
  // the reference by more than kRaise
  float mref = 0.f, mex = -INFINITY, om = 0.f;
  bool over = false;
  auto wave_scores = [&](auto I, int t, float (&sc)[4]) __attribute__((always_inline)) {
    const uint16_t* kb = KB(I);
    floatx4 sa = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + (KPW * wave + l16 % KPW) * D + 32 * ks + 8 * g4);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], sa, 0, 0, 0);
    }
    const int lim = c1 - (c0 + t * GK);  // keys of the tile inside the chunk: key < lim
    #pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = KPW * wave + (4 * g4 + e) % KPW < lim ? sa[e] * cs : -INFINITY;
  };
  // every key of the wave is held by some lanes (g4 < KPW / 4, all l16);
  // lanes l16 < 4 of those write one weight each
  auto weights = [&](auto I, const float (&sc)[4]) __attribute__((always_inline)) {
    float tm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if constexpr (KPW == 8) tm = fmaxf(tm, __shfl_xor(tm, 16));  // rows 0-3 and 4-7
    mex = fmaxf(mex, tm);
    over = over || tm > mref + kRaise;
    const int e4 = lane & 3;
    float sel = sc[0];
    #pragma unroll
    for (int e = 1; e < 4; ++e) sel = e4 == e ? sc[e] : sel;
    const float w = __builtin_amdgcn_exp2f(sel - mref);  // masked keys: 0
    const bool wr = l16 < 4 && g4 < KPW / 4;
    if (wr) SW(I)[KPW * wave + 4 * g4 + e4] = w;
    float ws = w;  // the sum over the wave's keys: lanes (e4, g4 < KPW / 4)
    ws += __shfl_xor(ws, 1);
    ws += __shfl_xor(ws, 2);
    if constexpr (KPW == 8) ws += __shfl_xor(ws, 16);
    om += ws;
  };

  // ---- staging: a lane of a G wave (C wave) holds dimension 32 brow + ql of
  // the keys (values) 16 ks + 8 g + e of the tile: w k (w v) as two bf16 terms
  // in registers, the A operand of its block row; the G waves also write the
  // raw keys transposed (KT), the B operand of every wave
  const int dim = 32 * brow + ql;
  float psum4[4];     // sum over this lane's keys of w k[dim] (w v[dim]), four chains
  bf16x8 ah[2][2], al[2][2];  // [tile parity][k-step]
  floatx16 acc[NB];
  auto stage_from = [&](auto I, const uint16_t* src) __attribute__((always_inline)) {
    constexpr int b = decltype(I)::value & 1;
    const float* w = SW(I);
    #pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const floatx4 w0 = *reinterpret_cast<const floatx4*>(w + 16 * ks + 8 * g);
      const floatx4 w1 = *reinterpret_cast<const floatx4*>(w + 16 * ks + 8 * g + 4);
      const float we[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      uint16_t raw[8];
      #pragma unroll
      for (int e = 0; e < 8; ++e) raw[e] = src[(16 * ks + 8 * g + e) * D + dim];
      // hi = p with its low 16 bits cleared (a bf16 value, exactly); lo = p - hi
      // (exact in fp32) rounded to bf16: hi + lo holds p to about 2^-16
      uint32_t hb[8];
      float lo[8];
      #pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = we[e] * __uint_as_float(static_cast<uint32_t>(raw[e]) << 16);
        psum4[e & 3] += p;
        hb[e] = __float_as_uint(p) & 0xffff0000u;
        lo[e] = p - __uint_as_float(hb[e]);
      }
      uint4 hp;
      hp.x = (hb[0] >> 16) | hb[1];
      hp.y = (hb[2] >> 16) | hb[3];
      hp.z = (hb[4] >> 16) | hb[5];
      hp.w = (hb[6] >> 16) | hb[7];
      ah[b][ks] = __builtin_bit_cast(bf16x8, hp);
      #pragma unroll
      for (int e = 0; e < 8; ++e) al[b][ks][e] = static_cast<__bf16>(lo[e]);
      if (kwave) {
        uint4 pk;
        pk.x = raw[0] | (static_cast<uint32_t>(raw[1]) << 16);
        pk.y = raw[2] | (static_cast<uint32_t>(raw[3]) << 16);
        pk.z = raw[4] | (static_cast<uint32_t>(raw[5]) << 16);
        pk.w = raw[6] | (static_cast<uint32_t>(raw[7]) << 16);
        // (brow is wave-uniform: the half is too)
        uint16_t* kt = brow < NB / 2 ? KT(I, IC<0>{}) : KT(I, IC<1>{});
        *reinterpret_cast<uint4*>(kt + (dim % (D / 2)) * KLD + 16 * ks + 8 * g) = pk;
      }
    }
  };
  auto stage = [&](auto I) __attribute__((always_inline)) {
    if (kwave) stage_from(I, KB(I));
    else stage_from(I, VB(I));
  };
  // products of the tile staged in parity I: block (brow, J) += A (hi, lo) x KT(J)
  auto gram = [&](auto I) __attribute__((always_inline)) {
    constexpr int b = decltype(I)::value & 1;
    const uint16_t* kta = KT(I, IC<0>{});
    const uint16_t* ktb = KT(I, IC<1>{});
    #pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 bb[NB];
      #pragma unroll
      for (int j = 0; j < NB; ++j)
        bb[j] = *reinterpret_cast<const bf16x8*>((j < NB / 2 ? kta : ktb) + (32 * (j % (NB / 2)) + ql) * KLD +
                                                 16 * ks + 8 * g);
      #pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[b][ks], bb[j], acc[j], 0, 0, 0);
      #pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[b][ks], bb[j], acc[j], 0, 0, 0);
    }
  };
  // step t (raw slot I = t % NR): copy tile t + NR - 1; products of tile
  // t - 1 (for t = 0 a zero product: zero A operands and a zeroed KT of
  // parity 1); scores and weights of tile t + 1 around the staging of tile t;
  // then this wave's copies of tile t + 2 have landed, and a barrier makes
  // everything visible
  auto step = [&](auto I, int t) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    copy(IC<(i + NR - 1) % NR>{}, t + NR - 1);
    gram(IC<(i + 1) % 2>{});
    float sc[4];
    wave_scores(IC<(i + 1) % NR>{}, t + 1, sc);
    stage(I);
    weights(IC<(i + 1) % NR>{}, sc);
    wait_copies_barrier<2 * (NR - 3)>();
  };

  // one pass over the chunk (a second only after an overflowing reference)
  bool second = false;
  float mall;  // the chunk's exact max
  for (;;) {
    #pragma unroll
    for (int e = 0; e < 4; ++e) psum4[e] = 0.f;
    #pragma unroll
    for (int j = 0; j < NB; ++j)
      #pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    #pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      #pragma unroll
      for (int e = 0; e < 8; ++e) {
        ah[1][ks][e] = static_cast<__bf16>(0.f);
        al[1][ks][e] = static_cast<__bf16>(0.f);
      }
    for (int c = tid; c < D / 2 * KLD / 8; c += SH::NT) {
      reinterpret_cast<uint4*>(kt1a)[c] = uint4{0, 0, 0, 0};
      reinterpret_cast<uint4*>(kt1b)[c] = uint4{0, 0, 0, 0};
    }
    copy(IC<0>{}, 0);
    copy(IC<1>{}, 1);
    copy(IC<2>{}, 2);
    copy(IC<3>{}, 3);
    copy(IC<4>{}, 4);
    wait_copies_barrier<2 * (NR - 2)>();  // tile 0 has landed
    {
      float sc[4];
      wave_scores(IC<0>{}, 0, sc);
      if (!second) {
        // the reference: tile 0's max (every wave: it also scales the sums at the end)
        float tm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        if constexpr (KPW == 8) tm = fmaxf(tm, __shfl_xor(tm, 16));
        if (lane == 0) sm0[wave] = tm;
        __syncthreads();
        mref = sm0[0];
        #pragma unroll
        for (int w = 1; w < SH::NW; ++w) mref = fmaxf(mref, sm0[w]);
      }
      weights(IC<0>{}, sc);
    }
    wait_copies_barrier<2 * (NR - 3)>();  // tile 1 has landed; weights of tile 0 visible
    for (int t0 = 0; t0 < ntlr; t0 += NR) {
      step(IC<0>{}, t0);
      step(IC<1>{}, t0 + 1);
      step(IC<2>{}, t0 + 2);
      step(IC<3>{}, t0 + 3);
      step(IC<4>{}, t0 + 4);
      step(IC<5>{}, t0 + 5);
    }
    gram(IC<1>{});  // the last tile, ntlr - 1 (odd)
    if (lane == 0) {
      sred[wave][0] = mex;
      sred[wave][1] = om;
      sred[wave][2] = over ? 1.f : 0.f;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no tile copy may still be in flight
    __syncthreads();
    mall = sred[0][0];
    float ovs = sred[0][2];
    #pragma unroll
    for (int w = 1; w < SH::NW; ++w) {
      mall = fmaxf(mall, sred[w][0]);
      ovs += sred[w][2];
    }
    if (!(ovs > 0.f)) break;  // uniform
    // again, against the chunk's exact max (no weight can pass 1 now)
    mref = mall;
    mex = -INFINITY;
    om = 0.f;
    over = false;
    second = true;
    __syncthreads();  // every wave has read sred
  }
  // everything against the chunk's exact max
  const float beta = __builtin_amdgcn_exp2f(mref - mall);
  float* pb = P.part + (static_cast<size_t>(bh) * P.S + sp) * SH::PSZ;
  if (tid == 0) {
    float o = 0.f;
    #pragma unroll
    for (int w = 0; w < SH::NW; ++w) o += sred[w][1];
    pb[0] = mall;
    pb[1] = o * beta;
    pb[2] = 0.f;
    pb[3] = 0.f;
  }
  // lanes ql and ql + 32 hold the two halves of one dimension's sum
  const float psum = (psum4[0] + psum4[1]) + (psum4[2] + psum4[3]);
  const float ps = (psum + __shfl_xor(psum, 32)) * beta;
  if (g == 0) pb[4 + (kwave ? 0 : D) + dim] = ps;
  // accumulator register r of lane (ql, g): row 8 (r / 4) + 4 g + r % 4 of the
  // block, column ql
  float* mb = pb + 4 + 2 * D + (kwave ? 0 : D * D);
  #pragma unroll
  for (int j = 0; j < NB; ++j)
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * brow + 8 * (r >> 2) + 4 * g + (r & 3);
      mb[row * D + 32 * j + ql] = acc[j][r] * beta;
    }
}

// The chunk partials of a head (S > 1) summed into one, each scaled by
// 2^(m_c - m) with m the head's max: the partial vector is linear in the
// weights except its max, which is replaced. Grid (slices of DT * 16 floats, BH).
template <int D>
__global__ __launch_bounds__(DT) void dec1_combine(Dec1Params P) {
  constexpr int PSZ = Dec1Shape<D>::PSZ;
  __shared__ float se[64], sm;
  const int bh = blockIdx.y, t = threadIdx.x;
  const float* base = P.part + static_cast<size_t>(bh) * P.S * PSZ;
  if (t < 64) {
    const float mc = t < P.S ? base[static_cast<size_t>(t) * PSZ] : -INFINITY;
    const float m = wave_max(mc);
    se[t] = t < P.S ? exp2f(mc - m) : 0.f;
    if (t == 0) sm = m;
  }
  __syncthreads();
  const float4* b4 = reinterpret_cast<const float4*>(base);
  float4* o4 = reinterpret_cast<float4*>(P.comb + static_cast<size_t>(bh) * PSZ);
  constexpr int NV = PSZ / 4;  // float4s of one partial
  #pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int f = blockIdx.x * (DT * 4) + u * DT + t;
    if (f >= NV) break;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    int c = 0;
    for (; c + 3 < P.S; c += 4) {  // four chunks' loads in flight
      float4 x[4];
      #pragma unroll
      for (int h = 0; h < 4; ++h) x[h] = b4[static_cast<size_t>(c + h) * NV + f];
      #pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float e = se[c + h];
        a.x += e * x[h].x; a.y += e * x[h].y; a.z += e * x[h].z; a.w += e * x[h].w;
      }
    }
    for (; c < P.S; ++c) {
      const float4 x = b4[static_cast<size_t>(c) * NV + f];
      const float e = se[c];
      a.x += e * x.x; a.y += e * x.y; a.z += e * x.z; a.w += e * x.w;
    }
    if (f == 0) a.x = sm;  // the max, not a sum
    o4[f] = a;
  }
}

// One head: Sigma_c = (G + G^T) / 2 - omega kbar kbar^T + lambda I, CG on
// Sigma_c x = mu = omega (kbar - q) in fp32, then the output and the optional
// outputs. Thread (row, part): row wave * RPW + lane % RPW of G and of C,
// columns [part CPP, (part + 1) CPP); the parts of a row sit in one wave and
// are summed with lane exchanges. G's and C's row segments are held in
// registers; p and x are shared through LDS; two reduction slots alternate,
// so a reduction needs one barrier.
template <int D>
__global__ __launch_bounds__(DT) void dec1_solve(Dec1Params P) {
  using SH = Dec1Shape<D>;
  constexpr int LG = D + 1, NP = DT / D, PSZ = SH::PSZ;
  constexpr int RPW = D / (DT / 64), CPP = D / NP;
  static_assert(RPW * NP == 64, "a wave holds whole rows");
  __shared__ float sG[D * LG];
  __shared__ float skb[D], swv[D], sx[D];
  __shared__ float red[2][DT / 64];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* src = P.S > 1 ? P.comb + static_cast<size_t>(bh) * PSZ : P.part + static_cast<size_t>(bh) * PSZ;
  const int row = wave * RPW + lane % RPW, part = lane / RPW;
  const bool own = part == 0;  // the lane that writes element `row`
  // every load in flight together: the moments, G (NG float4s per thread) and
  // this thread's segment of C's row
  constexpr int NG = D * D / 4 / DT;
  static_assert(NG * 4 * DT == D * D, "G must spread evenly over the threads");
  const float4* G4 = reinterpret_cast<const float4*>(src + 4 + 2 * D);
  const float4* C4 = reinterpret_cast<const float4*>(src + 4 + 2 * D + D * D) + (row * D + part * CPP) / 4;
  float4 ga[NG], cr[CPP / 4];
  #pragma unroll
  for (int u = 0; u < NG; ++u) ga[u] = G4[t + DT * u];
  #pragma unroll
  for (int u = 0; u < CPP / 4; ++u) cr[u] = C4[u];
  const float m = src[0], om = src[1];
  if (t < 2 * D) {
    const float v = src[4 + t];
    if (t < D) skb[t] = v / om;
    else swv[t - D] = v;
  }
  #pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int idx = 4 * (t + DT * u), i = idx / D, j = idx % D;
    sG[i * LG + j] = ga[u].x;
    sG[i * LG + j + 1] = ga[u].y;
    sG[i * LG + j + 2] = ga[u].z;
    sG[i * LG + j + 3] = ga[u].w;
  }
  __syncthreads();
  for (int idx = t; idx < D * D; idx += DT) {  // each pair i <= j by one thread
    const int i = idx / D, j = idx % D;
    if (j < i) continue;
    const float v = 0.5f * (sG[i * LG + j] + sG[j * LG + i]) - om * skb[i] * skb[j] + (i == j ? P.lambda : 0.f);
    sG[i * LG + j] = v;
    sG[j * LG + i] = v;
  }
  __syncthreads();
  float gr[CPP];
  #pragma unroll
  for (int c = 0; c < CPP; ++c) gr[c] = sG[row * LG + part * CPP + c];
  int rs = 0;  // reduction slot
  auto bsum = [&](float v) __attribute__((always_inline)) {
    v = wave_sum(v);
    if (lane == 0) red[rs][wave] = v;
    __syncthreads();
    float s = 0.f;
    #pragma unroll
    for (int w = 0; w < DT / 64; ++w) s += red[rs][w];
    rs ^= 1;
    return s;
  };
  // the sum over the parts of a row (lanes RPW apart)
  auto rowsum = [&](float v) __attribute__((always_inline)) {
    #pragma unroll
    for (int o = RPW; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
  };
  // CG; every lane of a row keeps that row's elements of x, r and p
  const float qv = __uint_as_float(static_cast<uint32_t>(P.q[static_cast<size_t>(bh) * D + row]) << 16);
  const float kb = skb[row];
  float x = 0.f, r = om * (kb - qv), pv = r;
  float rr = bsum(own ? r * r : 0.f);
  const float r0 = sqrtf(rr);
  const float thr = P.cg_rel_tol * r0;
  bool active = rr > 0.f && P.cg_max_iters > 0;
  int iters = 0;
  for (int it = 0; it < P.cg_max_iters && active; ++it) {  // `active` is block-uniform
    if (own) sx[row] = pv;
    __syncthreads();
    float ap = 0.f;
    #pragma unroll
    for (int c = 0; c < CPP; ++c) ap += gr[c] * sx[part * CPP + c];
    ap = rowsum(ap);
    const float pAp = bsum(own ? pv * ap : 0.f);
    if (!(pAp > 0.f)) break;  // breakdown: keep the iterate
    const float al = rr / pAp;
    x += al * pv;
    r -= al * ap;
    const float rrn = bsum(own ? r * r : 0.f);
    ++iters;
    if (sqrtf(rrn) <= thr || rrn == 0.f) {
      rr = rrn;
      break;
    }
    pv = r + (rrn / rr) * pv;
    rr = rrn;
  }
  const float kq = bsum(own ? (kb - qv) * x : 0.f);
  const float kx = bsum(own ? kb * x : 0.f);
  // C x from the registers
  if (own) sx[row] = x;
  __syncthreads();
  float cx = 0.f;
  #pragma unroll
  for (int u = 0; u < CPP / 4; ++u) {
    const float* xs = sx + part * CPP + 4 * u;
    cx += cr[u].x * xs[0] + cr[u].y * xs[1] + cr[u].z * xs[2] + cr[u].w * xs[3];
  }
  cx = rowsum(cx);
  if (own) {
    P.out[static_cast<size_t>(bh) * D + row] = (swv[row] * (1.f + kx) - cx) / om;
    // the pages' rho_i = rho_c / (1 + (kbar - q).rho_c)
    if (P.rho) P.rho[static_cast<size_t>(bh) * D + row] = x / (1.f + kq);
  }
  if (t == 0) {
    if (P.omega) P.omega[bh] = om;
    if (P.rowmax) P.rowmax[bh] = m * kLn2;
    if (P.cg_iters) P.cg_iters[bh] = iters;
    if (P.cg_resid) P.cg_resid[bh] = r0 > 0.f ? sqrtf(rr) / r0 : 0.f;
  }
}

size_t al256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

struct DecLayout {
  int S, L, SG, LG;
  size_t s, p1, gram, st, p4, total;  // byte offsets
};

DecLayout dec_layout(int BH, int n, int d) {
  DecLayout o{};
  // score, moment and output kernels: about eight workgroups per compute
  // unit, at least 64 keys per chunk
  int S = (2048 + BH - 1) / BH;
  S = std::max(1, std::min(S, std::min(64, (n + 63) / 64)));
  o.L = (n + S - 1) / S;
  o.S = (n + o.L - 1) / o.L;  // every chunk non-empty
  // Gram kernel: about two workgroups per compute unit, but each chunk Gram
  // (d^2 floats written, then read by the solve) no larger than a quarter of
  // the chunk's keys (L d values)
  int SG = (512 + BH - 1) / BH;
  SG = std::max(1, std::min(SG, std::min(64, n / (4 * d))));
  o.LG = (n + SG - 1) / SG;
  o.SG = (n + o.LG - 1) / o.LG;
  size_t off = 0;
  o.s = off;    off += al256(static_cast<size_t>(BH) * n * sizeof(float));
  o.p1 = off;   off += al256(static_cast<size_t>(BH) * o.S * (d + 2) * sizeof(float));
  o.gram = off; off += al256(static_cast<size_t>(BH) * o.SG * d * d * sizeof(float));
  o.st = off;   off += al256(static_cast<size_t>(BH) * (2 * d + 2) * sizeof(float));
  o.p4 = off;   off += al256(static_cast<size_t>(BH) * o.S * (d + 1) * sizeof(float));
  o.total = off;
  return o;
}

template <int D, typename T>
hipError_t launch_dec(const DecodeParams& p, hipStream_t stream) {
  const DecLayout ly = dec_layout(p.BH, p.n, D);
  char* ws = static_cast<char*>(p.workspace);
  DecParams P{};
  P.q = p.q; P.k = p.k; P.v = p.v; P.out = p.out;
  P.omega = p.omega; P.rho = p.rho; P.rowmax = p.rowmax; P.cg_iters = p.cg_iters; P.cg_resid = p.cg_resid;
  P.s = reinterpret_cast<float*>(ws + ly.s);
  P.p1 = reinterpret_cast<float*>(ws + ly.p1);
  P.gram = reinterpret_cast<float*>(ws + ly.gram);
  P.st = reinterpret_cast<float*>(ws + ly.st);
  P.p4 = reinterpret_cast<float*>(ws + ly.p4);
  P.BH = p.BH; P.n = p.n; P.S = ly.S; P.L = ly.L; P.SG = ly.SG; P.LG = ly.LG;
  P.lambda = p.lambda; P.cg_max_iters = p.cg_max_iters; P.cg_rel_tol = p.cg_rel_tol;
  const dim3 gs(ly.S, p.BH), gg(ly.SG, p.BH), gh(p.BH);
  hipLaunchKernelGGL((dec_moments<D, T>), gs, dim3(DT), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_main_begin && (e = hipEventRecord(p.ev_main_begin, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((dec_gram<D, T>), gg, dim3(DT), 0, stream, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.ev_main_end && (e = hipEventRecord(p.ev_main_end, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((dec_solve<D, T>), gh, dim3(DT), 0, stream, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((dec_output<D, T>), gs, dim3(DT), 0, stream, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((dec_finish<D>), gh, dim3(DT), 0, stream, P);
  return hipGetLastError();
}

struct Dec1Layout {
  int S, L;
  size_t comb, total;  // bytes: the chunk partials, then (S > 1) one combined partial per head
};

Dec1Layout dec1_layout(int BH, int n, int d) {
  Dec1Layout o{};
  // about one workgroup per compute unit (256), chunks of at least 512 keys,
  // at most 64 chunks per head
  int S = std::max(1, std::min(64, std::min(256 / BH, n / 512)));
  o.L = ((n + S - 1) / S + GK - 1) / GK * GK;
  o.S = (n + o.L - 1) / o.L;  // every chunk non-empty
  const size_t psz = (4 + 2 * static_cast<size_t>(d) + 2 * static_cast<size_t>(d) * d) * sizeof(float);
  o.comb = al256(static_cast<size_t>(BH) * o.S * psz);
  o.total = o.comb + (o.S > 1 ? al256(static_cast<size_t>(BH) * psz) : 0);
  return o;
}

template <int D>
hipError_t launch_dec1(const DecodeParams& p, hipStream_t stream) {
  const Dec1Layout ly = dec1_layout(p.BH, p.n, D);
  Dec1Params P{};
  P.q = static_cast<const uint16_t*>(p.q);
  P.k = static_cast<const uint16_t*>(p.k);
  P.v = static_cast<const uint16_t*>(p.v);
  P.out = p.out;
  P.omega = p.omega; P.rho = p.rho; P.rowmax = p.rowmax; P.cg_iters = p.cg_iters; P.cg_resid = p.cg_resid;
  P.part = static_cast<float*>(p.workspace);
  P.comb = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + ly.comb);
  P.BH = p.BH; P.n = p.n; P.S = ly.S; P.L = ly.L;
  P.lambda = p.lambda; P.cg_max_iters = p.cg_max_iters; P.cg_rel_tol = p.cg_rel_tol;
  hipError_t e;
  if (p.ev_main_begin && (e = hipEventRecord(p.ev_main_begin, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((dec1_chunk<D>), dim3(ly.S, p.BH), dim3(Dec1Shape<D>::NT), 0, stream, P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.ev_main_end && (e = hipEventRecord(p.ev_main_end, stream)) != hipSuccess) return e;
  if (ly.S > 1) {
    constexpr int NV = Dec1Shape<D>::PSZ / 4;
    hipLaunchKernelGGL((dec1_combine<D>), dim3((NV + 4 * DT - 1) / (4 * DT), p.BH), dim3(DT), 0, stream, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dec1_solve<D>), dim3(p.BH), dim3(DT), 0, stream, P);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int d) { return d == 64 || d == 128; }

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode entry point: a file-scope device array
// of kDecodeScratchBytes that every GPU the library runs on holds until the
// process ends. Host code must not use `scratch` itself as a device address
// (in host code it names a host-side stand-in); decode_scratch() looks up the
// array's address on the current device once and keeps it per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int BH, int n, int d, int dtype) {
  return dtype == LLA_DTYPE_BF16 ? dec1_layout(BH, n, d).total : dec_layout(BH, n, d).total;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.dtype == LLA_DTYPE_BF16) return p.d == 128 ? launch_dec1<128>(p, stream) : launch_dec1<64>(p, stream);
  return p.d == 128 ? launch_dec<128, float>(p, stream) : launch_dec<64, float>(p, stream);
}

}  // namespace lla
