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

#include <type_traits>

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


typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// round two floats to fp16 (nearest even) and add their rounded values to acc
// with one packed dot product against (1, 1): acc + h0 + h1 exactly in fp32
__device__ __forceinline__ half2v pack_sum(float a, float b, float& acc) {
  half2v h;
  h[0] = static_cast<_Float16>(a);
  h[1] = static_cast<_Float16>(b);
  const half2v one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  acc = __builtin_amdgcn_fdot2(h, one, acc, false);
  return h;
}

__device__ __forceinline__ float pair_sum(float v) { return v + __shfl_xor(v, 32); }
__device__ __forceinline__ float pair_max(float v) { return fmaxf(v, __shfl_xor(v, 32)); }

struct Workspace {
  float* partial;   // [BH][nchunk][2]: max row ||.||^2 of q and k; of v
  _Float16* kr;     // [BH][npad][D]      s k, d index permuted by swz16
  _Float16* kt;     // [BH][npad/32][D][32] s k transposed, key index permuted
  _Float16* vt;     // [BH][npad/32][D][32] sv v transposed, key index permuted
  float* xs;        // CG iterates: per workgroup BQ x D fp32, lane-contiguous
  float* kbs;       // fp32 kbar, same layout
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
  p += t;
  const size_t nqb = static_cast<size_t>((n + BQ - 1) / BQ);
  const size_t sl = align256(static_cast<size_t>(BH) * nqb * BQ * d * sizeof(float));
  w.xs = reinterpret_cast<float*>(p);
  p += sl;
  w.kbs = reinterpret_cast<float*>(p);
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
  float* xs;         // CG iterate slab, [blocks][4 waves][d/8 float4 chunks][64 lanes]
  float* kbs;        // fp32 kbar slab, same layout
  int BH, n, nchunk, nblk;
  float lambda;
  int cg_max_iters;
  float cg_rel_tol;
};

// LDS tiles. The K-row tile holds BK rows of D fp16 (the d index already
// permuted by swz16 within 16-element chunks); the transposed tile holds D
// rows of BK fp16 keys. Neither is padded: the 16-byte chunk c of a row sits
// at chunk position c ^ chunk_xor(row) instead, which spreads the rows that one
// 16-lane group reads in the same operand step over distinct LDS banks.
template <int D>
__device__ __forceinline__ int kr_chunk_xor(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int kt_chunk_xor(int row) { return (row >> 2) & 3; }

// Copy key tile `kt` of this head straight from global memory into the LDS
// tiles (global_load_lds: each wave instruction fills 1 KiB of LDS, lane l
// its l-th 16 bytes; the source address of each lane applies the chunk
// permutation). Completion is awaited by the next __syncthreads().
template <int D>
__device__ __forceinline__ void load_tile_to_lds(const _Float16* kr_head, const _Float16* t_head,
                                                 int kt, _Float16* sKr, _Float16* sKt, int wave,
                                                 int lane) {
  constexpr int CPR = D / 8;          // 16-byte chunks per K row
  constexpr int RPI = 64 / CPR;       // K rows per wave instruction
  constexpr int NI = D / 64;          // instructions per wave for each tile
  #pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int inst = wave * NI + u;
    const int row = inst * RPI + lane / CPR;
    const int c = (lane % CPR) ^ kr_chunk_xor<D>(row);
    const _Float16* src = kr_head + (static_cast<size_t>(kt) * BK + row) * D + c * 8;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(src),
        (__attribute__((address_space(3))) void*)(sKr + inst * 512), 16, 0, 0);
  }
  #pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int inst = wave * NI + u;
    const int row = inst * 16 + lane / 4;
    const int c = (lane % 4) ^ kt_chunk_xor(row);
    const _Float16* src = t_head + static_cast<size_t>(kt) * D * BK + row * BK + c * 8;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(src),
        (__attribute__((address_space(3))) void*)(sKt + inst * 512), 16, 0, 0);
  }
}

// Work order. Workgroups are handed to the eight XCDs (each with its own L2)
// in turn: block b runs on XCD b % 8. When the head count divides by 8, each
// XCD gets its own heads and walks them one after the other, every head's
// query blocks longest causal prefix first, so the key tiles that an XCD's
// workgroups stream are those of about one head at a time and stay in its L2.
// Otherwise the order is longest prefix first across all heads.
constexpr int kXcds = 8;
__device__ __forceinline__ void block_coords(int b, int BH, int nqb, int* qb, int* bh) {
  if (BH % kXcds == 0) {
    const int xcd = b % kXcds, j = b / kXcds;
    const int heads_per_xcd = BH / kXcds;
    *bh = xcd * heads_per_xcd + j / nqb;
    *qb = nqb - 1 - j % nqb;
  } else {
    *qb = nqb - 1 - b / BH;
    *bh = b % BH;
  }
}

template <int D, bool SPLIT_U>
__global__ __launch_bounds__(NT) void lla_mfma_main(MainParams P) {
  constexpr int NKS = D / 16;  // k-steps over d
  constexpr int NMB = D / 32;  // 32-row blocks over d
  __shared__ __align__(16) _Float16 sKr[2][BK * D];
  __shared__ __align__(16) _Float16 sKt[2][D * BK];
  __shared__ __align__(16) half8 sKb[NT / 64][NKS][64];     // kbar, fp16, operand order
  __shared__ __align__(16) floatx4 sR[NT / 64][NMB * 4][64];  // CG residual r, fp32
  __shared__ float sScale[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int n = P.n;
  const int nqb = (n + BQ - 1) / BQ;
  int qb, bh;
  block_coords(static_cast<int>(blockIdx.x), P.BH, nqb, &qb, &bh);
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
    load_tile_to_lds<D>(kr_head, t_head, 0, sKr[0], sKt[0], wave, lane);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < ntiles) load_tile_to_lds<D>(kr_head, t_head, kt + 1, sKr[buf ^ 1], sKt[buf ^ 1], wave, lane);
      if (wave_busy && kt <= wlast) tile(kt, buf);
      __syncthreads();
    }
  };

  // this lane's operand fragments in the LDS tiles
  const int krx = kr_chunk_xor<D>(ql), ktx = kt_chunk_xor(ql);
  auto kr_frag = [&](int buf, int t) __attribute__((always_inline)) {
    return *reinterpret_cast<const half8*>(sKr[buf] + ql * D + 8 * ((2 * t + g) ^ krx));
  };
  auto kt_frag = [&](int buf, int mb, int h) __attribute__((always_inline)) {
    return *reinterpret_cast<const half8*>(sKt[buf] + (32 * mb + ql) * BK + 8 * ((2 * h + g) ^ ktx));
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
    half8 kf[NKS], tf[2 * NMB];
    #pragma unroll
    for (int t = 0; t < NKS; ++t) kf[t] = kr_frag(buf, t);
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int h = 0; h < 2; ++h) tf[2 * mb + h] = kt_frag(buf, mb, h);
    floatx16 sacc = mfma(kf[0], qop[0], floatx16{});
    #pragma unroll
    for (int t = 1; t < NKS; ++t) sacc = mfma(kf[t], qop[t], sacc);
    const int lim = kmax - kt * BK;  // keys <= lim are visible
    half8 wb[2];
    auto body = [&](auto masked) __attribute__((always_inline)) {
      float sc[16];
      float tmax = -INFINITY;
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[r] * c2s;
        if constexpr (decltype(masked)::value) {
          if (key_of(r) > lim) x = -INFINITY;
        }
        sc[r] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = pair_max(tmax);
      const float mnew = fmaxf(m2, tmax);
      // a query with every key so far masked (only queries past the end) keeps
      // its running max at -inf; then nothing is accumulated for it
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(m2 - mref);
      float wsum = 0.f;
      #pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const half2v hw = pack_sum(fast_exp2(sc[r] - mref), fast_exp2(sc[r + 1] - mref), wsum);
        wb[r >> 3][r & 7] = hw[0];
        wb[r >> 3][(r & 7) + 1] = hw[1];
      }
      om = om * alpha + wsum;
      m2 = mnew;
      if (alpha != 1.f)
        #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[mb] *= alpha;
    };
    if (wave_full && kt < wlast)
      body(std::false_type{});
    else
      body(std::true_type{});
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int h = 0; h < 2; ++h) acc[mb] = mfma(tf[2 * mb + h], wb[h], acc[mb]);
  }, wave_any);
  om = pair_sum(om);
  if (!qvalid) m2 = 0.f;

  // --------------------------- CG set-up -------------------------------
  // Per query: kbar = mu~ / omega, r0 = mu = mu~ - omega q, x0 = 0. Nothing
  // large stays in registers across a key sweep: r lives in LDS (fp32), x and
  // the fp32 kbar in lane-contiguous workspace slabs, and the CG matvec uses
  // kbar rounded to fp16 from LDS as its expansion point. The matvec is exact
  // for any expansion point c used consistently in U = w (K d - c.d) and in
  // the correction -(sum U) c (the shift of c.d cancels through sum U), so
  // rounding kbar only moves the centre: Sigma_c becomes
  // Sigma_c + omega (kbar - c)(kbar - c)^T, a rank-one change of relative size
  // 2^-24. Phase 3 uses the fp32 kbar.
  const size_t slab = (static_cast<size_t>(blockIdx.x) * (NT / 64) + wave) * (NMB * 4 * 64);
  floatx4* xs = reinterpret_cast<floatx4*>(P.xs) + slab;
  floatx4* kbs = reinterpret_cast<floatx4*>(P.kbs) + slab;
  float rr = 0.f;
  {
    const float inv_om = qvalid ? 1.f / om : 0.f;
    half8 kb16[NKS];
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        floatx4 kb, rc;
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          const float mt = acc[mb][r];
          const float qv = static_cast<float>(qop[2 * mb + (r >> 3)][r & 7]);
          kb[b] = mt * inv_om;
          kb16[2 * mb + (r >> 3)][r & 7] = static_cast<_Float16>(kb[b]);
          rc[b] = qvalid ? mt - om * qv : 0.f;
          rr += rc[b] * rc[b];
        }
        kbs[(mb * 4 + a) * 64 + lane] = kb;
        xs[(mb * 4 + a) * 64 + lane] = floatx4{0.f, 0.f, 0.f, 0.f};
        sR[wave][mb * 4 + a][lane] = rc;
      }
    #pragma unroll
    for (int t = 0; t < NKS; ++t) sKb[wave][t][lane] = kb16[t];
  }
  rr = pair_sum(rr);
  const float r0n = sqrtf(rr);
  const float thr = P.cg_rel_tol * r0n;
  bool active = qvalid && rr > 0.f && P.cg_max_iters > 0;
  int iters = 0;

  // fp16 kbar . op for an operand-ordered fp16 vector
  auto kbar_dot = [&](const half8 (&op)[NKS]) __attribute__((always_inline)) {
    float acc_ = 0.f;
    #pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const half8 kb = sKb[wave][t][lane];
      #pragma unroll
      for (int c = 0; c < 8; ++c) acc_ += static_cast<float>(kb[c]) * static_cast<float>(op[t][c]);
    }
    return pair_sum(acc_);
  };

  // direction d = fp16(p / sp), sp a power of two with |p / sp| <= 1
  half8 dop[NKS];
  float sp = 1.f;
  {
    float rv[NMB][16];
    float mx = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 rc = sR[wave][mb * 4 + a][lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          rv[mb][4 * a + b] = rc[b];
          mx = fmaxf(mx, fabsf(rc[b]));
        }
      }
    sp = pow2_ceil(pair_max(mx));
    const float inv = 1.f / sp;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) dop[2 * mb + (r >> 3)][r & 7] = static_cast<_Float16>(rv[mb][r] * inv);
  }
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
    floatx16 tinit;
    #pragma unroll
    for (int r = 0; r < 16; ++r) tinit[r] = -kbd;
    sweep(kt_head, [&](int kt, int buf) __attribute__((always_inline)) {
      half8 kf[NKS], tf[2 * NMB];
      #pragma unroll
      for (int t = 0; t < NKS; ++t) kf[t] = kr_frag(buf, t);
      #pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        #pragma unroll
        for (int h = 0; h < 2; ++h) tf[2 * mb + h] = kt_frag(buf, mb, h);
      // S = K Q^T; T = K d^T - kbar.d (the shift enters as the accumulator's
      // initial value, so U = w T needs one multiply per element)
      floatx16 sacc = mfma(kf[0], qop[0], floatx16{});
      floatx16 tacc = mfma(kf[0], dop[0], tinit);
      #pragma unroll
      for (int t = 1; t < NKS; ++t) {
        sacc = mfma(kf[t], qop[t], sacc);
        tacc = mfma(kf[t], dop[t], tacc);
      }
      half8 ub[2], ul[2];
      const int lim = kmax - kt * BK;  // keys <= lim are visible
      auto make_u = [&](auto masked) __attribute__((always_inline)) {
        #pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float w0 = fast_exp2(fmaf(sacc[r], c2s, -m2));
          float w1 = fast_exp2(fmaf(sacc[r + 1], c2s, -m2));
          if constexpr (decltype(masked)::value) {
            if (key_of(r) > lim) w0 = 0.f;
            if (key_of(r + 1) > lim) w1 = 0.f;
          }
          const float u0 = w0 * tacc[r], u1 = w1 * tacc[r + 1];
          const half2v hu = pack_sum(u0, u1, usum);
          ub[r >> 3][r & 7] = hu[0];
          ub[r >> 3][(r & 7) + 1] = hu[1];
          if constexpr (SPLIT_U) {
            const half2v lo = pack_sum(u0 - static_cast<float>(hu[0]),
                                       u1 - static_cast<float>(hu[1]), usum);
            ul[r >> 3][r & 7] = lo[0];
            ul[r >> 3][(r & 7) + 1] = lo[1];
          }
        }
      };
      // the causal mask only bites on the wave's diagonal tile (wave-uniform)
      if (wave_full && kt < wlast)
        make_u(std::false_type{});
      else
        make_u(std::true_type{});
      #pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        #pragma unroll
        for (int h = 0; h < 2; ++h) {
          acc[mb] = mfma(tf[2 * mb + h], ub[h], acc[mb]);
          if constexpr (SPLIT_U) acc[mb] = mfma(tf[2 * mb + h], ul[h], acc[mb]);
        }
    }, wave_busy);
    usum = pair_sum(usum);

    // CG step (registers only in this stretch): Sigma_c d = Y - (sum U) c +
    // lambda d with c the fp16 kbar; exact line search along d; then the next
    // direction p = r + beta sp d, renormalised and rounded to fp16.
    float rv[NMB][16], ad[NMB][16];
    float dAd = 0.f, rd = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 rc = sR[wave][mb * 4 + a][lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) rv[mb][4 * a + b] = rc[b];
      }
      #pragma unroll
      for (int h = 0; h < 2; ++h) {
        const half8 kb = sKb[wave][2 * mb + h][lane];
        #pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int r = 8 * h + c;
          const float dv = static_cast<float>(dop[2 * mb + h][c]);
          const float v = acc[mb][r] - usum * static_cast<float>(kb[c]) + lam_s * dv;
          ad[mb][r] = v;
          dAd += dv * v;
          rd += rv[mb][r] * dv;
        }
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
        if (step) rv[mb][r] -= al * ad[mb][r];
        rrn += rv[mb][r] * rv[mb][r];
      }
    if (step) {
      #pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
          floatx4 xc = xs[(mb * 4 + a) * 64 + lane];
          floatx4 rc;
          #pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int r = 4 * a + b;
            xc[b] += al * static_cast<float>(dop[2 * mb + (r >> 3)][r & 7]);
            rc[b] = rv[mb][r];
          }
          xs[(mb * 4 + a) * 64 + lane] = xc;
          sR[wave][mb * 4 + a][lane] = rc;
        }
    }
    rrn = pair_sum(rrn);
    bool cont = false;
    if (step) {
      ++iters;
      cont = !(sqrtf(rrn) <= thr || rrn == 0.f);
    }
    // lanes that stopped keep their state; the pair exchanges run in every lane
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
    float xv[NMB][16];
    float mx = 0.f, nn = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 xc = xs[(mb * 4 + a) * 64 + lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          xv[mb][4 * a + b] = xc[b];
          mx = fmaxf(mx, fabsf(xc[b]));
          nn += xc[b] * xc[b];
        }
      }
    srho = pow2_ceil(pair_max(mx));
    nn = pair_sum(nn);
    const float inv = 1.f / srho;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float xsc = xv[mb][r] * inv;
        const _Float16 h = static_cast<_Float16>(xsc);
        rhi[2 * mb + (r >> 3)][r & 7] = h;
        rlo[2 * mb + (r >> 3)][r & 7] = static_cast<_Float16>(xsc - static_cast<float>(h));
      }
    float kd = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 kb = kbs[(mb * 4 + a) * 64 + lane];
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
  // racc starts at -kbar.rho' / srho (srho is a power of two: exact), so
  // (k - kbar).rho' = srho racc and a / sA = w (inv_sA - srho inv_sA racc)
  const float a_slope = -srho * inv_sA;
  floatx16 rinit;
  #pragma unroll
  for (int r = 0; r < 16; ++r) rinit[r] = -kr_dot / srho;
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  float den = 0.f;
  sweep(vt_head, [&](int kt, int buf) __attribute__((always_inline)) {
    half8 kf[NKS], tf[2 * NMB];
    #pragma unroll
    for (int t = 0; t < NKS; ++t) kf[t] = kr_frag(buf, t);
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int h = 0; h < 2; ++h) tf[2 * mb + h] = kt_frag(buf, mb, h);
    // S = K Q^T; R = K (hi + lo)^T - kbar.rho' / srho, the shift entering as
    // the accumulator's initial value; then a = w (1 - srho R) / sA
    floatx16 sacc = mfma(kf[0], qop[0], floatx16{});
    floatx16 racc = mfma(kf[0], rhi[0], rinit);
    racc = mfma(kf[0], rlo[0], racc);
    #pragma unroll
    for (int t = 1; t < NKS; ++t) {
      sacc = mfma(kf[t], qop[t], sacc);
      racc = mfma(kf[t], rhi[t], racc);
      racc = mfma(kf[t], rlo[t], racc);
    }
    const int lim = kmax - kt * BK;
    half8 ab[2];
    auto body = [&](auto masked) __attribute__((always_inline)) {
      #pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float w0 = fast_exp2(fmaf(sacc[r], c2s, -m2));
        float w1 = fast_exp2(fmaf(sacc[r + 1], c2s, -m2));
        if constexpr (decltype(masked)::value) {
          if (key_of(r) > lim) w0 = 0.f;
          if (key_of(r + 1) > lim) w1 = 0.f;
        }
        const float a0 = w0 * fmaf(racc[r], a_slope, inv_sA);
        const float a1 = w1 * fmaf(racc[r + 1], a_slope, inv_sA);
        const half2v ha = pack_sum(a0, a1, den);
        ab[r >> 3][r & 7] = ha[0];
        ab[r >> 3][(r & 7) + 1] = ha[1];
      }
    };
    if (wave_full && kt < wlast)
      body(std::false_type{});
    else
      body(std::true_type{});
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int h = 0; h < 2; ++h) acc[mb] = mfma(tf[2 * mb + h], ab[h], acc[mb]);
  }, wave_any);
  den = pair_sum(den);

  if (!qvalid) return;
  const size_t orow = static_cast<size_t>(bh) * n + qi;
  const float ob = 1.f / (den * sv);
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
    }
  if (P.rho) {
    // the pages' rho_i = rho_c / (1 + (kbar - q).rho_c), in input units
    float qx = 0.f, kx = 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 kb = kbs[(mb * 4 + a) * 64 + lane];
        const floatx4 xc = xs[(mb * 4 + a) * 64 + lane];
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          qx += static_cast<float>(qop[2 * mb + (r >> 3)][r & 7]) * xc[b];
          kx += kb[b] * xc[b];
        }
      }
    // (both lanes of the pair are valid here, so the exchange is well defined)
    qx = pair_sum(qx);
    kx = pair_sum(kx);
    const float rs = s / (1.f + (kx - qx));
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 xc = xs[(mb * 4 + a) * 64 + lane];
        const int dim = 32 * mb + 8 * a + 4 * g;
        *reinterpret_cast<float4*>(P.rho + orow * D + dim) =
            make_float4(xc[0] * rs, xc[1] * rs, xc[2] * rs, xc[3] * rs);
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
  m.xs = w.xs;
  m.kbs = w.kbs;
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
  const size_t nqb = static_cast<size_t>((n + BQ - 1) / BQ);
  return align256(static_cast<size_t>(BH) * nchunk * 2 * sizeof(float)) +
         3 * align256(static_cast<size_t>(BH) * npad * d * sizeof(_Float16)) +
         2 * align256(static_cast<size_t>(BH) * nqb * BQ * d * sizeof(float));
}

hipError_t launch_mfma(const FwdParams& p, hipStream_t stream) {
  if (p.n > (1 << 21) || p.BH > 0x7fffffff) return hipErrorInvalidValue;
  if (p.d == 128) return launch_d<128>(p, stream);
  if (p.d == 64) return launch_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lla
