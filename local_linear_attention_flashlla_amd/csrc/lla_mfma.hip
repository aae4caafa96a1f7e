// Matrix-core kernel for the causal LLA forward pass: bf16 inputs, d in
// {64, 128}, gfx950 (CDNA4) v_mfma_f32_32x32x16_f16.
//
// The blocked three-phase forward of "Local Linear Attention: reading notes"
// (section 2.2, Algorithm 1) runs as one persistent workgroup per block of
// BQ = 128 queries of one (batch, head), four waves of 32 queries each:
//   phase 1: for each 32-key tile, S = K Q^T on MFMA, online row max, weights
//            w = exp(S - m), omega += sum w, mu~ += K^T W on MFMA
//            (Eqs. (10)-(11));
//   phase 2: matrix-free CG on Sigma_c rho = mu (the system centred at
//            kbar = mu~ / omega, see include/lla.h): per iteration one sweep
//            over the key tiles forms S = K Q^T and T = K D^T with one shared
//            K fragment, U = w (T - kbar.d), Y += K^T U on MFMA; then
//            Sigma_c d = Y - (sum U) kbar + lambda d and a CG step per query
//            (Eq. (12) with the expansion point moved to kbar);
//   phase 3: S = K Q^T and R = K rho^T on MFMA, a = w (1 - (k - kbar).rho),
//            O += V^T A on MFMA, out = O / sum a (Eq. (8)).
//
// Numerics. Inputs are bf16; bf16 values convert exactly to fp16 when in
// range, so the matrix cores run fp16 x fp16 -> fp32 (same dense rate as bf16,
// eight times finer rounding for the CG operands). A prepass scales q, k of
// each head by one power of two s (and v by sv) so that every row norm is at
// most 128: scaling by a power of two is exact, keeps fp16 far from overflow
// and is undone exactly (scores use c / s^2, the ridge lambda s^2). Per query,
// the CG direction is carried as fp16 d = p / sp with sp a power of two; the
// CG step uses an exact line search along d, so rounding the direction only
// perturbs conjugacy, never the residual recurrence. rho enters phase 3 as two
// fp16 terms (hi + lo, ~22 bits).
//
// Register layout. All per-query state lives in the MFMA accumulator layout
// with the query along lanes: lane l serves query l % 32 of its wave, and lane
// half g = l / 32 holds the d-components 32 mb + 8 a + 4 g + b (b < 4, a < 4,
// mb < d/32) in accumulator register 16 mb + 4 a + b. Per-query dot products
// are an in-lane sum plus one exchange with lane l ^ 32. The same lane also
// supplies the query's fp16 operand for the next product straight from these
// registers: the contraction index is permuted inside every 16-element chunk
// (bits 2 and 3 swapped), and the LDS copies of the K rows (d index) and of
// the transposed K / V tiles (key index) are stored with the same permutation,
// so every operand fragment is a single 16-byte LDS read and no data moves
// between lanes.

#include <hip/hip_runtime.h>
#include <math.h>

#include "lla_internal.h"
#include "../../include/lla.h"

namespace lla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = 128;     // queries per workgroup
constexpr int BK = 32;      // keys per tile
constexpr int NT = 256;     // threads per workgroup (4 waves)
constexpr int NORM_ROWS = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRowNormCap = 128.f;

// bits 2 and 3 of the index inside a 16-element chunk swapped (an involution)
__host__ __device__ constexpr int swz16(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

__device__ __forceinline__ float bf16_to_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// smallest power of two >= m for m > 0 (1 for m <= 0 or NaN)
__device__ __forceinline__ float pow2_ceil(float m) {
  if (!(m > 0.f)) return 1.f;
  uint32_t b = __float_as_uint(m);
  uint32_t e = b >> 23;
  if (e == 0) return 1.1754943508222875e-38f;
  if (b & 0x7fffffu) e += 1;
  if (e > 254) e = 254;
  return __uint_as_float(e << 23);
}

// largest power of two <= m for m > 0
__device__ __forceinline__ float pow2_floor(float m) {
  uint32_t e = __float_as_uint(m) >> 23;
  if (e == 0) e = 1;
  if (e > 254) e = 254;
  return __uint_as_float(e << 23);
}

__device__ __forceinline__ floatx16 mfma(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float pair_sum(float v) { return v + __shfl_xor(v, 32); }
__device__ __forceinline__ float pair_max(float v) { return fmaxf(v, __shfl_xor(v, 32)); }

struct Workspace {
  float* partial;   // [BH][nchunk][2]: max row ||.||^2 of q and k; of v
  _Float16* kr;     // [BH][npad][D]      s k, d index permuted by swz16
  _Float16* kt;     // [BH][npad/32][D][32] s k transposed, key index permuted
  _Float16* vt;     // [BH][npad/32][D][32] sv v transposed, key index permuted
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Workspace carve(void* base, int BH, int n, int d) {
  const int nchunk = (n + NORM_ROWS - 1) / NORM_ROWS;
  const size_t npad = static_cast<size_t>((n + BK - 1) / BK) * BK;
  char* p = static_cast<char*>(base);
  Workspace w;
  w.partial = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(BH) * nchunk * 2 * sizeof(float));
  const size_t t = align256(static_cast<size_t>(BH) * npad * d * sizeof(_Float16));
  w.kr = reinterpret_cast<_Float16*>(p);
  p += t;
  w.kt = reinterpret_cast<_Float16*>(p);
  p += t;
  w.vt = reinterpret_cast<_Float16*>(p);
  return w;
}

// The per-head power-of-two scales, from the row-norm partial maxima.
__device__ __forceinline__ void head_scales(const float* partial, int bh, int nchunk, float* s,
                                            float* sv) {
  float mqk = 0.f, mv = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    mqk = fmaxf(mqk, partial[(static_cast<size_t>(bh) * nchunk + c) * 2 + 0]);
    mv = fmaxf(mv, partial[(static_cast<size_t>(bh) * nchunk + c) * 2 + 1]);
  }
  const float a = sqrtf(mqk), b = sqrtf(mv);
  *s = a > 0.f ? fminf(fmaxf(pow2_floor(kRowNormCap / a), 0x1p-60f), 0x1p60f) : 1.f;
  *sv = b > 0.f ? fminf(fmaxf(pow2_floor(kRowNormCap / b), 0x1p-60f), 0x1p60f) : 1.f;
}

// ---------------------------------------------------------------------------
// Prepass 1: per (head, chunk of 256 rows) the largest squared row norm of q
// and k together, and of v.
template <int D>
__global__ __launch_bounds__(NT) void prep_norms(const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ k,
                                                 const uint16_t* __restrict__ v, int n, int nchunk,
                                                 float* __restrict__ partial) {
  const int bh = blockIdx.x, chunk = blockIdx.y;
  const int i = chunk * NORM_ROWS + threadIdx.x;
  float mqk = 0.f, mv = 0.f;
  if (i < n) {
    const size_t off = (static_cast<size_t>(bh) * n + i) * D;
    float sq = 0.f, sk = 0.f, sw = 0.f;
    for (int c = 0; c < D; c += 8) {
      const uint4 a = *reinterpret_cast<const uint4*>(q + off + c);
      const uint4 b = *reinterpret_cast<const uint4*>(k + off + c);
      const uint4 e = *reinterpret_cast<const uint4*>(v + off + c);
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w},
                     ev[4] = {e.x, e.y, e.z, e.w};
      for (int u = 0; u < 4; ++u) {
        float x0 = bf16_to_f(av[u] & 0xffffu), x1 = bf16_to_f(av[u] >> 16);
        sq += x0 * x0 + x1 * x1;
        x0 = bf16_to_f(bv[u] & 0xffffu); x1 = bf16_to_f(bv[u] >> 16);
        sk += x0 * x0 + x1 * x1;
        x0 = bf16_to_f(ev[u] & 0xffffu); x1 = bf16_to_f(ev[u] >> 16);
        sw += x0 * x0 + x1 * x1;
      }
    }
    mqk = fmaxf(sq, sk);
    mv = sw;
  }
  for (int o = 32; o > 0; o >>= 1) {
    mqk = fmaxf(mqk, __shfl_xor(mqk, o));
    mv = fmaxf(mv, __shfl_xor(mv, o));
  }
  __shared__ float red[2][NT / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = mqk;
    red[1][wave] = mv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = red[0][0], b = red[1][0];
    for (int w = 1; w < NT / 64; ++w) {
      a = fmaxf(a, red[0][w]);
      b = fmaxf(b, red[1][w]);
    }
    // a NaN/Inf input makes the scale meaningless but must not make it 0
    partial[(static_cast<size_t>(bh) * nchunk + chunk) * 2 + 0] = a;
    partial[(static_cast<size_t>(bh) * nchunk + chunk) * 2 + 1] = b;
  }
}

// Prepass 2: per (head, 32-key block) write s k in fp16 as permuted rows and
// as a permuted transposed tile, and sv v as a permuted transposed tile.
template <int D>
__global__ __launch_bounds__(NT) void prep_convert(const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, int n,
                                                   int nchunk, int nblk,
                                                   const float* __restrict__ partial,
                                                   _Float16* __restrict__ kr,
                                                   _Float16* __restrict__ kt,
                                                   _Float16* __restrict__ vt) {
  const int bh = blockIdx.x, kb = blockIdx.y;
  __shared__ float sK[BK][D + 1];
  __shared__ float sV[BK][D + 1];
  __shared__ float sc[2];
  if (threadIdx.x == 0) head_scales(partial, bh, nchunk, &sc[0], &sc[1]);
  __syncthreads();
  const float s = sc[0], sv = sc[1];
  for (int e = threadIdx.x; e < BK * D; e += NT) {
    const int r = e / D, c = e % D;
    const int j = kb * BK + r;
    float a = 0.f, b = 0.f;
    if (j < n) {
      const size_t off = (static_cast<size_t>(bh) * n + j) * D + c;
      a = bf16_to_f(k[off]) * s;
      b = bf16_to_f(v[off]) * sv;
    }
    sK[r][c] = a;
    sV[r][c] = b;
  }
  __syncthreads();
  const size_t npad = static_cast<size_t>(nblk) * BK;
  for (int e = threadIdx.x; e < BK * D; e += NT) {
    const int r = e / D, pos = e % D;
    const int src = (pos & ~15) | swz16(pos & 15);
    kr[(static_cast<size_t>(bh) * npad + kb * BK + r) * D + pos] = static_cast<_Float16>(sK[r][src]);
  }
  const size_t tb = (static_cast<size_t>(bh) * nblk + kb) * D;
  for (int e = threadIdx.x; e < BK * D; e += NT) {
    const int dim = e / BK, pos = e % BK;
    const int key = (pos & 16) | swz16(pos & 15);
    kt[(tb + dim) * BK + pos] = static_cast<_Float16>(sK[key][dim]);
    vt[(tb + dim) * BK + pos] = static_cast<_Float16>(sV[key][dim]);
  }
}

// ---------------------------------------------------------------------------
struct MainParams {
  const uint16_t* q;
  float* out;
  float* omega;
  float* rho;
  float* rowmax;
  int32_t* cg_iters;
  float* cg_resid;
  const float* partial;
  const _Float16* kr;
  const _Float16* kt;
  const _Float16* vt;
  int BH, n, nchunk, nblk;
  float lambda;
  int cg_max_iters;
  float cg_rel_tol;
};

template <int D>
struct TileLoader {
  static constexpr int KRS = D + 8;        // LDS row stride of the K-row tile (halves)
  static constexpr int KTS = BK + 8;       // LDS row stride of the transposed tiles (halves)
  static constexpr int NR = BK * D / 8 / NT;  // 16-byte chunks per thread, row tile
  static constexpr int NTR = D * BK / 8 / NT; // 16-byte chunks per thread, transposed tile
  u32x4 r[NR];
  u32x4 t[NTR];

  __device__ __forceinline__ void load(const _Float16* kr_head, const _Float16* t_head, int kt) {
    const int tid = threadIdx.x;
    #pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int e = tid + NT * u;
      const int row = e / (D / 8), c8 = e % (D / 8);
      r[u] = *reinterpret_cast<const u32x4*>(kr_head + (static_cast<size_t>(kt) * BK + row) * D + c8 * 8);
    }
    #pragma unroll
    for (int u = 0; u < NTR; ++u) {
      const int e = tid + NT * u;
      t[u] = *reinterpret_cast<const u32x4*>(t_head + static_cast<size_t>(kt) * D * BK + e * 8);
    }
  }
  __device__ __forceinline__ void store(_Float16* sKr, _Float16* sKt) const {
    const int tid = threadIdx.x;
    #pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int e = tid + NT * u;
      const int row = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<u32x4*>(sKr + row * KRS + c8 * 8) = r[u];
    }
    #pragma unroll
    for (int u = 0; u < NTR; ++u) {
      const int e = tid + NT * u;
      const int row = e / (BK / 8), c = e % (BK / 8);
      *reinterpret_cast<u32x4*>(sKt + row * KTS + c * 8) = t[u];
    }
  }
};

template <int D, bool SPLIT_U>
__global__ __launch_bounds__(NT) void lla_mfma_main(MainParams P) {
  constexpr int NKS = D / 16;  // k-steps over d
  constexpr int NMB = D / 32;  // 32-row blocks over d
  using TL = TileLoader<D>;
  constexpr int KRS = TL::KRS, KTS = TL::KTS;
  __shared__ __align__(16) _Float16 sKr[2][BK * KRS];
  __shared__ __align__(16) _Float16 sKt[2][D * KTS];
  __shared__ __align__(16) floatx4 sKb[NT / 64][NMB * 4][64];
  __shared__ float sScale[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int n = P.n;
  const int nqb = (n + BQ - 1) / BQ;
  const int qb = nqb - 1 - static_cast<int>(blockIdx.x) / P.BH;  // longest prefix first
  const int bh = static_cast<int>(blockIdx.x) % P.BH;
  const int i0 = qb * BQ;
  const int kend = min(n, i0 + BQ);
  const int ntiles = (kend + BK - 1) / BK;
  const int qi = i0 + 32 * wave + ql;
  const bool qvalid = qi < n;
  const int kmax = qvalid ? qi : -1;      // last key this lane's query sees
  const int wfirst = i0 + 32 * wave;      // first query of the wave
  const bool wave_any = wfirst < n;
  const bool wave_full = wfirst + 31 < n;
  const int wlast = wave_any ? min(ntiles - 1, (wfirst + 31) / BK) : -1;  // last tile of the wave

  if (tid == 0) head_scales(P.partial, bh, P.nchunk, &sScale[0], &sScale[1]);
  __syncthreads();
  const float s = sScale[0], sv = sScale[1];
  const float c2s = kLog2e / sqrtf(static_cast<float>(D)) / (s * s);
  const float lam_s = P.lambda * s * s;

  const _Float16* kr_head = P.kr + static_cast<size_t>(bh) * P.nblk * BK * D;
  const _Float16* kt_head = P.kt + static_cast<size_t>(bh) * P.nblk * BK * D;
  const _Float16* vt_head = P.vt + static_cast<size_t>(bh) * P.nblk * BK * D;

  // Q operand of this lane's query: slot (t, c) holds s q[16 t + 8 (c >> 2) + 4 g + (c & 3)]
  half8 qop[NKS];
  {
    const uint16_t* qrow = P.q + (static_cast<size_t>(bh) * n + (qvalid ? qi : 0)) * D;
    #pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const uint2 lo = *reinterpret_cast<const uint2*>(qrow + 16 * t + 4 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(qrow + 16 * t + 8 + 4 * g);
      const uint32_t w4[4] = {lo.x, lo.y, hi.x, hi.y};
      #pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float a = qvalid ? bf16_to_f(w4[u] & 0xffffu) * s : 0.f;
        const float b = qvalid ? bf16_to_f(w4[u] >> 16) * s : 0.f;
        qop[t][2 * u] = static_cast<_Float16>(a);
        qop[t][2 * u + 1] = static_cast<_Float16>(b);
      }
    }
  }

  // The key sweep: tiles 0 .. ntiles-1 of this head, double-buffered through
  // LDS; `tile(kt, buf)` runs on the waves whose queries see tile kt.
  auto sweep = [&](const _Float16* t_head, auto&& tile, bool wave_busy) __attribute__((always_inline)) {
    TL ld;
    ld.load(kr_head, t_head, 0);
    ld.store(sKr[0], sKt[0]);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < ntiles) ld.load(kr_head, t_head, kt + 1);
      if (wave_busy && kt <= wlast) tile(kt, buf);
      if (kt + 1 < ntiles) ld.store(sKr[buf ^ 1], sKt[buf ^ 1]);
      __syncthreads();
    }
  };

  // key index (within the tile) of accumulator register r of this lane
  auto key_of = [&](int r) __attribute__((always_inline)) { return 8 * (r >> 2) + 4 * g + (r & 3); };

  floatx16 acc[NMB];
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  // ------------------------------ phase 1 ------------------------------
  float m2 = -INFINITY;  // running row max of the log2-scaled scores
  float om = 0.f;        // partial row sum (this half of the keys)
  sweep(kt_head, [&](int kt, int buf) __attribute__((always_inline)) {
    floatx16 sacc;
    #pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    const _Float16* a_row = sKr[buf] + ql * KRS + 8 * g;
    #pragma unroll
    for (int t = 0; t < NKS; ++t)
      sacc = mfma(*reinterpret_cast<const half8*>(a_row + 16 * t), qop[t], sacc);
    const bool full = wave_full && kt < wlast;
    float sc[16];
    float tmax = -INFINITY;
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = sacc[r] * c2s;
      if (!full && kt * BK + key_of(r) > kmax) x = -INFINITY;
      sc[r] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = pair_max(tmax);
    const float mnew = fmaxf(m2, tmax);
    const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m2 - mnew);
    half8 wb[2];
    float wsum = 0.f;
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float w = (sc[r] == -INFINITY) ? 0.f : fast_exp2(sc[r] - mnew);
      const _Float16 wh = static_cast<_Float16>(w);
      wb[r >> 3][r & 7] = wh;
      wsum += static_cast<float>(wh);
    }
    om = om * alpha + wsum;
    m2 = mnew;
    if (alpha != 1.f)
      #pragma unroll
      for (int mb = 0; mb < NMB; ++mb) acc[mb] *= alpha;
    const _Float16* t_row = sKt[buf] + ql * KTS + 8 * g;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[mb] = mfma(*reinterpret_cast<const half8*>(t_row + 32 * mb * KTS + 16 * h), wb[h], acc[mb]);
  }, wave_any);
  om = pair_sum(om);
  if (!qvalid) m2 = 0.f;

  // --------------------------- CG set-up -------------------------------
  // kbar = mu~ / omega (kept in LDS), r0 = mu = mu~ - omega q, x0 = 0.
  float xr[NMB][16], rv[NMB][16];
  float rr = 0.f;
  {
    const float inv_om = qvalid ? 1.f / om : 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        floatx4 kb;
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          const float mt = acc[mb][r];
          const float qv = static_cast<float>(qop[2 * mb + (r >> 3)][r & 7]);
          kb[b] = mt * inv_om;
          rv[mb][r] = qvalid ? mt - om * qv : 0.f;
          xr[mb][r] = 0.f;
          rr += rv[mb][r] * rv[mb][r];
        }
        sKb[wave][mb * 4 + a][lane] = kb;
      }
  }
  rr = pair_sum(rr);
  const float r0n = sqrtf(rr);
  const float thr = P.cg_rel_tol * r0n;
  bool active = qvalid && rr > 0.f && P.cg_max_iters > 0;
  int iters = 0;

  // direction d = fp16(p / sp), sp a power of two with |p / sp| <= 1
  half8 dop[NKS];
  float sp = 1.f;
  auto set_direction = [&](const float (&p)[NMB][16]) {
    float mx = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(p[mb][r]));
    sp = pow2_ceil(pair_max(mx));
    const float inv = 1.f / sp;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) dop[2 * mb + (r >> 3)][r & 7] = static_cast<_Float16>(p[mb][r] * inv);
  };
  auto kbar_dot = [&](const half8 (&op)[NKS]) {
    float acc_ = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 kb = sKb[wave][mb * 4 + a][lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          acc_ += kb[b] * static_cast<float>(op[2 * mb + (r >> 3)][r & 7]);
        }
      }
    return pair_sum(acc_);
  };
  set_direction(rv);
  float kbd = kbar_dot(dop);

  // ------------------------------ phase 2 ------------------------------
  for (int it = 0; it < P.cg_max_iters; ++it) {
    if (!__syncthreads_or(active ? 1 : 0)) break;
    const bool wave_busy = __any(active ? 1 : 0);
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
    float usum = 0.f;
    sweep(kt_head, [&](int kt, int buf) __attribute__((always_inline)) {
      floatx16 sacc, tacc;
      #pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = tacc[r] = 0.f;
      const _Float16* a_row = sKr[buf] + ql * KRS + 8 * g;
      #pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const half8 a = *reinterpret_cast<const half8*>(a_row + 16 * t);
        sacc = mfma(a, qop[t], sacc);
        tacc = mfma(a, dop[t], tacc);
      }
      const bool full = wave_full && kt < wlast;
      half8 ub[2], ul[2];
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        float w = fast_exp2(sacc[r] * c2s - m2);
        if (!full && kt * BK + key_of(r) > kmax) w = 0.f;
        const float u = w * (tacc[r] - kbd);
        const _Float16 uh = static_cast<_Float16>(u);
        ub[r >> 3][r & 7] = uh;
        usum += static_cast<float>(uh);
        if constexpr (SPLIT_U) {
          const _Float16 lo = static_cast<_Float16>(u - static_cast<float>(uh));
          ul[r >> 3][r & 7] = lo;
          usum += static_cast<float>(lo);
        }
      }
      const _Float16* t_row = sKt[buf] + ql * KTS + 8 * g;
      #pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        #pragma unroll
        for (int h = 0; h < 2; ++h) {
          const half8 a = *reinterpret_cast<const half8*>(t_row + 32 * mb * KTS + 16 * h);
          acc[mb] = mfma(a, ub[h], acc[mb]);
          if constexpr (SPLIT_U) acc[mb] = mfma(a, ul[h], acc[mb]);
        }
    }, wave_busy);
    usum = pair_sum(usum);
    // Sigma_c d = Y - (sum U) kbar + lambda d; exact line search along d.
    float dAd = 0.f, rd = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 kb = sKb[wave][mb * 4 + a][lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          const float dv = static_cast<float>(dop[2 * mb + (r >> 3)][r & 7]);
          const float ad = acc[mb][r] - usum * kb[b] + lam_s * dv;
          acc[mb][r] = ad;
          dAd += dv * ad;
          rd += rv[mb][r] * dv;
        }
      }
    dAd = pair_sum(dAd);
    rd = pair_sum(rd);
    const bool step = active && dAd > 0.f;
    const float al = step ? rd / dAd : 0.f;
    float rrn = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dv = static_cast<float>(dop[2 * mb + (r >> 3)][r & 7]);
        if (step) {
          xr[mb][r] += al * dv;
          rv[mb][r] -= al * acc[mb][r];
        }
        rrn += rv[mb][r] * rv[mb][r];
      }
    rrn = pair_sum(rrn);
    bool cont = false;
    if (step) {
      ++iters;
      cont = !(sqrtf(rrn) <= thr || rrn == 0.f);
    }
    // next direction p = r + beta p_prev with p_prev = sp d, normalised to a
    // power of two and rounded to fp16; lanes that stopped keep their state.
    // The pair exchanges run in every lane.
    const float be = (step && rr > 0.f) ? rrn / rr * sp : 0.f;
    float mx = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r)
        mx = fmaxf(mx, fabsf(rv[mb][r] + be * static_cast<float>(dop[2 * mb + (r >> 3)][r & 7])));
    const float sp_new = pow2_ceil(pair_max(mx));
    const float inv_sp = 1.f / sp_new;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 2 * mb + (r >> 3), c = r & 7;
        const float pv = rv[mb][r] + be * static_cast<float>(dop[t][c]);
        if (cont) dop[t][c] = static_cast<_Float16>(pv * inv_sp);
      }
    if (cont) sp = sp_new;
    const float kbdn = kbar_dot(dop);
    if (cont) kbd = kbdn;
    if (step) rr = rrn;
    active = cont;
  }

  // ------------------------------ phase 3 ------------------------------
  // rho' = x as two fp16 terms: x = srho (hi + lo)
  half8 rhi[NKS], rlo[NKS];
  float srho, kr_dot, inv_sA;
  {
    float mx = 0.f, nn = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        mx = fmaxf(mx, fabsf(xr[mb][r]));
        nn += xr[mb][r] * xr[mb][r];
      }
    srho = pow2_ceil(pair_max(mx));
    nn = pair_sum(nn);
    const float inv = 1.f / srho;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float xs = xr[mb][r] * inv;
        const _Float16 h = static_cast<_Float16>(xs);
        rhi[2 * mb + (r >> 3)][r & 7] = h;
        rlo[2 * mb + (r >> 3)][r & 7] = static_cast<_Float16>(xs - static_cast<float>(h));
      }
    float kd = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 kb = sKb[wave][mb * 4 + a][lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          const int t = 2 * mb + (r >> 3), c = r & 7;
          kd += kb[b] * (static_cast<float>(rhi[t][c]) + static_cast<float>(rlo[t][c]));
        }
      }
    kr_dot = pair_sum(kd) * srho;
    // |(k - kbar).rho'| <= 2 * 128 * ||rho'||, so a / sA stays within [-1, 1]
    inv_sA = 1.f / pow2_ceil(1.f + 2.f * kRowNormCap * sqrtf(nn));
  }
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  float den = 0.f;
  sweep(vt_head, [&](int kt, int buf) __attribute__((always_inline)) {
    floatx16 sacc, racc;
    #pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = racc[r] = 0.f;
    const _Float16* a_row = sKr[buf] + ql * KRS + 8 * g;
    #pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const half8 a = *reinterpret_cast<const half8*>(a_row + 16 * t);
      sacc = mfma(a, qop[t], sacc);
      racc = mfma(a, rhi[t], racc);
      racc = mfma(a, rlo[t], racc);
    }
    const bool full = wave_full && kt < wlast;
    half8 ab[2];
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      float w = fast_exp2(sacc[r] * c2s - m2);
      if (!full && kt * BK + key_of(r) > kmax) w = 0.f;
      const float av = w * (1.f - (racc[r] * srho - kr_dot)) * inv_sA;
      const _Float16 ah = static_cast<_Float16>(av);
      ab[r >> 3][r & 7] = ah;
      den += static_cast<float>(ah);
    }
    const _Float16* t_row = sKt[buf] + ql * KTS + 8 * g;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[mb] = mfma(*reinterpret_cast<const half8*>(t_row + 32 * mb * KTS + 16 * h), ab[h], acc[mb]);
  }, wave_any);
  den = pair_sum(den);

  if (!qvalid) return;
  const size_t orow = static_cast<size_t>(bh) * n + qi;
  const float ob = 1.f / (den * sv);
  float qx = 0.f, kx = 0.f;
  if (P.rho) {
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 kb = sKb[wave][mb * 4 + a][lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          qx += static_cast<float>(qop[2 * mb + (r >> 3)][r & 7]) * xr[mb][r];
          kx += kb[b] * xr[mb][r];
        }
      }
  }
  // (both lanes of the pair are valid here, so the exchange is well defined)
  qx = pair_sum(qx);
  kx = pair_sum(kx);
  const float rs = s / (1.f + (kx - qx));  // the pages' rho_i in input units
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dim = 32 * mb + 8 * a + 4 * g;
      float4 o;
      o.x = acc[mb][4 * a + 0] * ob;
      o.y = acc[mb][4 * a + 1] * ob;
      o.z = acc[mb][4 * a + 2] * ob;
      o.w = acc[mb][4 * a + 3] * ob;
      *reinterpret_cast<float4*>(P.out + orow * D + dim) = o;
      if (P.rho) {
        float4 p4;
        p4.x = xr[mb][4 * a + 0] * rs;
        p4.y = xr[mb][4 * a + 1] * rs;
        p4.z = xr[mb][4 * a + 2] * rs;
        p4.w = xr[mb][4 * a + 3] * rs;
        *reinterpret_cast<float4*>(P.rho + orow * D + dim) = p4;
      }
    }
  if (g == 0) {
    if (P.omega) P.omega[orow] = om;
    if (P.rowmax) P.rowmax[orow] = m2 * kLn2;
    if (P.cg_iters) P.cg_iters[orow] = iters;
    if (P.cg_resid) P.cg_resid[orow] = r0n > 0.f ? sqrtf(rr) / r0n : 0.f;
  }
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  const int n = p.n;
  const int nchunk = (n + NORM_ROWS - 1) / NORM_ROWS;
  const int nblk = (n + BK - 1) / BK;
  const Workspace w = carve(p.workspace, p.BH, n, D);
  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  const uint16_t* k = static_cast<const uint16_t*>(p.k);
  const uint16_t* v = static_cast<const uint16_t*>(p.v);
  hipLaunchKernelGGL(prep_norms<D>, dim3(p.BH, nchunk), dim3(NT), 0, stream, q, k, v, n, nchunk,
                     w.partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prep_convert<D>, dim3(p.BH, nblk), dim3(NT), 0, stream, k, v, n, nchunk, nblk,
                     w.partial, w.kr, w.kt, w.vt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  MainParams m{};
  m.q = q;
  m.out = p.out;
  m.omega = p.omega;
  m.rho = p.rho;
  m.rowmax = p.rowmax;
  m.cg_iters = p.cg_iters;
  m.cg_resid = p.cg_resid;
  m.partial = w.partial;
  m.kr = w.kr;
  m.kt = w.kt;
  m.vt = w.vt;
  m.BH = p.BH;
  m.n = n;
  m.nchunk = nchunk;
  m.nblk = nblk;
  m.lambda = p.lambda;
  m.cg_max_iters = p.cg_max_iters;
  m.cg_rel_tol = p.cg_rel_tol;
  const long long blocks = static_cast<long long>((n + BQ - 1) / BQ) * p.BH;
  if (p.ev_main_begin) {
    e = hipEventRecord(p.ev_main_begin, stream);
    if (e != hipSuccess) return e;
  }
  if (p.flags & LLA_FLAG_SPLIT_U)
    hipLaunchKernelGGL((lla_mfma_main<D, true>), dim3(static_cast<unsigned>(blocks)), dim3(NT), 0,
                       stream, m);
  else
    hipLaunchKernelGGL((lla_mfma_main<D, false>), dim3(static_cast<unsigned>(blocks)), dim3(NT), 0,
                       stream, m);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_main_end) return hipEventRecord(p.ev_main_end, stream);
  return hipSuccess;
}

}  // namespace

bool mfma_supported(int dtype, int d) { return dtype == LLA_DTYPE_BF16 && (d == 64 || d == 128); }

size_t mfma_workspace_bytes(int BH, int n, int d) {
  const int nchunk = (n + NORM_ROWS - 1) / NORM_ROWS;
  const size_t npad = static_cast<size_t>((n + BK - 1) / BK) * BK;
  return align256(static_cast<size_t>(BH) * nchunk * 2 * sizeof(float)) +
         3 * align256(static_cast<size_t>(BH) * npad * d * sizeof(_Float16));
}

hipError_t launch_mfma(const FwdParams& p, hipStream_t stream) {
  if (p.n > (1 << 21) || p.BH > 0x7fffffff) return hipErrorInvalidValue;
  if (p.d == 128) return launch_d<128>(p, stream);
  if (p.d == 64) return launch_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lla
