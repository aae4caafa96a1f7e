// Matrix-core kernels for the gradient of the causal LLA forward pass: bf16
// inputs, d in {64, 128}, gfx950.
//
// "Local Linear Attention: reading notes" (section 2.2, the remark on
// training, and appendix D) says that the backward pass of LLA needs further
// linear systems per query but prints none. The gradient here is implicit
// differentiation of the forward as the matrix-core forward computes it,
// around the weighted key mean kbar_i = sum_j w_ij k_j / omega_i (Eqs. (6)-(8)
// rewritten, as in the forward's CG system): per query i, with g = dL/db_i,
// c_j = k_j - kbar, u = kbar - q, A_j = 1 - c_j.rho_c, beta_j = g.(v_j - vbar),
//
//   b = vbar - C rho_c,  C = sum_j (w_j / omega) v_j c_j^T,
//   Sigma_c rho_c = omega u,  Sigma_c = sum_j w_j c_j c_j^T + lambda I;
//   h = C^T g,  adjoint solve  Sigma_c y = h;
//   e_j = beta_j / omega - c_j.y,  tau = h.rho_c / omega - y.u;
//   dL/dw_j = A_j e_j + tau;  dL/ds_j = w_j dL/dw_j, plus at the key j* that
//   attains the row max m (w = exp(s - m)) minus the row's sum of those,
//   which equals lambda y.rho_c (scaling every weight is scaling lambda);
//   dq_i  = c sum_j dL/ds_j k_j + omega y,
//   dk_j += c dL/ds_j q - w_j (A_j y + e_j rho_c),
//   dv_j += (w_j A_j / omega) g,   c = 1/sqrt(d).
//
// Kernels, in launch order (the first two and the CG are the forward's own):
//   prepasses + moment kernel   per-head scales, fp16 key/value tiles, kbar,
//                               omega, row max m per query;
//   prep_vrows                  fp16 value tiles in row layout;
//   bwd_sweep<0>  (per query)   one sweep over the key tiles: scores
//                               S = K Q^T, G = V (s_g g)^T, U = w (G - g.b),
//                               Y += K^T U on MFMA, the argmax key j*;
//                               writes the adjoint right-hand side s h;
//   CG kernel                   Sigma_c y = h (same stop rule as the forward);
//   bwd_rows      (per query)   the per-query constants and operand tiles
//                               below, from the forward's rho_c and the
//                               adjoint solution;
//   bwd_sweep<1>  (per query)   one sweep: S, R = K rho_c^T, Yp = K y^T, G;
//                               dL/ds on the vector ALU; dq += K^T dL/ds,
//                               the max's share taken off at the end;
//   bwd_keys      (per key)     one sweep over the query tiles, keys along
//                               lanes: the same four score products, then
//                               dk += [q; y; rho_c]^T [c dL/ds; -w A; -w e]
//                               and dv += (-g/omega)^T (-w A) on bf16 MFMA.
//
// Numerics. Score-side products use fp16 operands with per-query power-of-two
// scales (as in the forward; rho_c as two fp16 terms). The dk/dv products run
// in bf16 (fp32 range: no scaling, 8-bit significands, unbiased rounding),
// whose error averages over the queries a key sees. dq's product uses fp16
// with a per-query power-of-two scale chosen from a bound on |dL/ds|.

#include <hip/hip_runtime.h>
#include <math.h>

#include "lla_internal.h"
#include "../../include/lla.h"
#include "lla_mfma_common.h"

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx16 mfma_bf(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per 32-query tile one contiguous record: seven fp16 tiles in the row
// layout of the key tiles (chunk-major, d index permuted), the fp32
// per-query constants [16][32] (padded to 4 KiB), then four bf16 tiles in the
// transposed layout (query index permuted). rho_c, y and the cotangent g
// enter the score products as two fp16 terms (hi + lo) each: where the local
// fit nearly interpolates (a short prefix, small lambda), rho_c is of order
// 1/lambda and e = beta/omega - c.y of order lambda, a difference of O(1)
// terms, so dk = ... - w e rho_c multiplies the rounding of y or g by
// 1/lambda; with one fp16 term each that costs percents there.
enum { T_QR = 0, T_RH, T_RL, T_YH, T_YL, T_GH, T_GL, kNRowTiles };
enum { T_QT = 0, T_YT, T_RT, T_GT, kNTransTiles };
enum {
  C_SINIT = 0,  // -m (log2 units): initial value of the score accumulator
  C_RINIT,      // -kbar.rho_c / srho
  C_RSLOPE,     // -srho: A = 1 + C_RSLOPE * R
  C_YINIT,      // -kbar.y / sy
  C_GINIT,      // -s_g s_v g.vbar
  C_EG,         // 1 / (s_g s_v omega): e = G C_EG + Yp C_EY
  C_EY,         // -sy
  C_TAU,        // tau
  C_MSUM,       // the row sum of w dL/dw, -lambda y.rho_c
  C_JSTAR,      // maximising key (int bits), -1 for a padding row
  C_F,          // power-of-two scale of dL/ds in the dq product
  C_OMS,        // omega s: dq gets omega y = C_OMS * y_s
  C_DQS,        // c / (f s): dq gets C_DQS * sum_j f dL/ds_j s k_j
  kNConst = 16
};
template <int D>
constexpr size_t tile_bytes() { return static_cast<size_t>(BK) * D * 2; }
constexpr size_t kCstBytes = 4096;  // constants [16][32] fp32, padded
template <int D>
constexpr size_t cst_off() { return kNRowTiles * tile_bytes<D>(); }
template <int D>
constexpr size_t row_part() { return cst_off<D>() + kCstBytes; }  // rows + constants
template <int D>
constexpr size_t rec_bytes() { return row_part<D>() + kNTransTiles * tile_bytes<D>(); }
static_assert(row_part<128>() % 4096 == 0 && row_part<64>() % 4096 == 0 &&
                  (kNTransTiles * tile_bytes<64>()) % 4096 == 0,
              "both parts of a record split into 1 KiB copies evenly over four waves");

struct BwdWorkspace {
  _Float16* vr;   // [BH][nblk][BK*D] sv v, row layout
  char* rec;      // [BH][nblk] per-query-tile records
  int32_t* jstar; // [BH][n] maximising key per query
  float* gvb;     // [BH][n] g . vbar per query (the weighted mean of g . v_j)
};

size_t rec_bytes_d(int d) { return d == 128 ? rec_bytes<128>() : rec_bytes<64>(); }

BwdWorkspace carve_bwd(void* base, int BH, int n, int d) {
  const size_t nblk = static_cast<size_t>((n + BK - 1) / BK);
  char* p = static_cast<char*>(base) + mfma_workspace_bytes(BH, n, d);
  BwdWorkspace w;
  w.vr = reinterpret_cast<_Float16*>(p);
  p += align256(static_cast<size_t>(BH) * nblk * BK * d * sizeof(_Float16));
  w.rec = p;
  p += align256(static_cast<size_t>(BH) * nblk * rec_bytes_d(d));
  w.jstar = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(BH) * n * sizeof(int32_t));
  w.gvb = reinterpret_cast<float*>(p);
  return w;
}

// ---------------------------------------------------------------------------
// Value tiles in the row layout of the key tiles (for G = V g^T).
template <int D>
__global__ __launch_bounds__(NT) void prep_vrows(const uint16_t* __restrict__ v, int n, int nchunk,
                                                 int nblk, const float* __restrict__ partial,
                                                 _Float16* __restrict__ vr) {
  const int bh = blockIdx.x, kb = blockIdx.y;
  __shared__ float sV[BK][D + 1];
  __shared__ float sc[2];
  if (threadIdx.x < 64) {
    float a, b;
    head_scales(partial, bh, nchunk, threadIdx.x, &a, &b);
    if (threadIdx.x == 0) {
      sc[0] = a;
      sc[1] = b;
    }
  }
  __syncthreads();
  const float sv = sc[1];
  for (int e = threadIdx.x; e < BK * D; e += NT) {
    const int r = e / D, c = e % D;
    const int j = kb * BK + r;
    sV[r][c] = j < n ? bf16_to_f(v[(static_cast<size_t>(bh) * n + j) * D + c]) * sv : 0.f;
  }
  __syncthreads();
  const size_t tb = (static_cast<size_t>(bh) * nblk + kb) * BK * D;
  for (int e = threadIdx.x; e < BK * D; e += NT) {
    const int c = e / (8 * BK), r = (e / 8) % BK, pos = 8 * c + e % 8;
    const int src = (pos & ~15) | swz16(pos & 15);
    vr[tb + e] = static_cast<_Float16>(sV[r][src]);
  }
}

// ---------------------------------------------------------------------------
struct SweepParams {
  const uint16_t* q;
  const uint16_t* k;
  const float* out;
  const float* dout;
  const float* partial;
  const _Float16* kr;
  const _Float16* kt;
  const _Float16* vr;
  float* xs;
  float* kbs;
  float* rs;
  float* qs;
  const char* rec;
  int32_t* jstar;
  float* gvb;
  float* dq;
  int BH, n, nchunk, nblk, nq32;
};

// Query-major sweep over the key tiles of each block of 128 queries (four
// waves of 32; the query along lanes as in the forward's kernels), tiles in
// three LDS buffers with one barrier per tile.
//   MODE 0: the adjoint right-hand side and the maximising key;
//   MODE 1: dq.
template <int D, int MODE>
__global__ __launch_bounds__(NT) void bwd_sweep(SweepParams P) {
  constexpr int NKS = D / 16, NMB = D / 32, NW = NT / 64, BQW = 32 * NW;
  // The dq sweep runs a two-stage pipeline over three tile buffers; the
  // right-hand-side sweep keeps two workgroups per CU instead (its second
  // accumulator set would cost the second one) and runs the stages in turn.
  constexpr bool PIPE = MODE == 1;
  constexpr int NB = PIPE ? 3 : 2;
  constexpr int NCPT = 3 * ((D / 16 + NW - 1) / NW);  // copy instructions per tile and wave
  static_assert(NCPT == 6 || NCPT == 3, "vmcnt below");
  __shared__ __align__(16) _Float16 sKr[NB][BK * D];
  __shared__ __align__(16) _Float16 sVr[NB][BK * D];
  __shared__ __align__(16) _Float16 sKt[NB][BK * D];
  __shared__ float sScale[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;
  const int n = P.n;
  const int nqb = (n + BQW - 1) / BQW;
  int qb, bh;
  block_coords(static_cast<int>(blockIdx.x), P.BH, nqb, &qb, &bh);
  const int i0 = qb * BQW;
  const int kend = min(n, i0 + BQW);
  const int ntiles = (kend + BK - 1) / BK;
  const int qi = i0 + 32 * wave + ql;
  const bool qvalid = qi < n;
  const int wfirst = i0 + 32 * wave;
  const bool wave_any = wfirst < n;
  const int wlast = wave_any ? min(ntiles - 1, wfirst / BK) : -1;

  if (tid < 64) {
    float a, b;
    head_scales(P.partial, bh, P.nchunk, tid, &a, &b);
    if (tid == 0) {
      sScale[0] = a;
      sScale[1] = b;
    }
  }
  __syncthreads();
  const float s = sScale[0], sv = sScale[1];

  const size_t head_elems = static_cast<size_t>(P.nblk) * BK * D;
  const uint32_t head_bytes = static_cast<uint32_t>(head_elems * sizeof(_Float16));
  const __amdgpu_buffer_rsrc_t kr_head = make_rsrc(P.kr + bh * head_elems, head_bytes);
  const __amdgpu_buffer_rsrc_t kt_head = make_rsrc(P.kt + bh * head_elems, head_bytes);
  const __amdgpu_buffer_rsrc_t vr_head = make_rsrc(P.vr + bh * head_elems, head_bytes);
  const size_t wslot = static_cast<size_t>(bh) * P.nq32 + (i0 >> 5) + wave;
  const __amdgpu_buffer_rsrc_t xs = make_rsrc(P.xs + wslot * (32 * D), 32 * D * 4);
  const __amdgpu_buffer_rsrc_t kbs = make_rsrc(P.kbs + wslot * (32 * D), 32 * D * 4);
  const __amdgpu_buffer_rsrc_t rsl = make_rsrc(P.rs + wslot * (32 * D), 32 * D * 4);
  const float* qst = P.qs + wslot * 128;
  const size_t orow = static_cast<size_t>(bh) * n + (qvalid ? qi : 0);

  auto kr_frag_at = [&](const _Float16* b, int t) __attribute__((always_inline)) {
    return *reinterpret_cast<const half8*>(b + ((2 * t + g) * BK + ql) * 8);
  };
  auto kt_frag_at = [&](const _Float16* b, int mb, int h) __attribute__((always_inline)) {
    return *reinterpret_cast<const half8*>(b + ((2 * h + g) * D + 32 * mb + ql) * 8);
  };
  auto key_of = [&](int r) __attribute__((always_inline)) { return 8 * (r >> 2) + 4 * g + (r & 3); };

  // per-query operands (B operands of the score products) and constants
  half8 qop[NKS], gop[NKS], glo[NKS];
  // (dq takes y as one fp16 term: its error there stays at the 1e-4 level even
  // where the fit nearly interpolates; dk needs two, see bwd_keys)
  half8 rh[MODE == 1 ? NKS : 1], rl[MODE == 1 ? NKS : 1], yop[MODE == 1 ? NKS : 1];
  float sinit_v = 0.f, ginit_v = 0.f;
  float sg = 1.f, om = 0.f, gb_row = 0.f;
  float c_rinit = 0.f, c_rslope = 0.f, c_yinit = 0.f, c_eg = 0.f, c_ey = 0.f, c_tau = 0.f,
        c_f = 0.f, c_oms = 0.f, c_dqs = 0.f;
  int jst = -1;
  if constexpr (MODE == 0) {
    const float qsc = kLog2e / sqrtf(static_cast<float>(D)) / s;
    const uint16_t* qrow = P.q + orow * D;
    const float* grow = P.dout + orow * D;
    const float* brow = P.out + orow * D;
    float gv[NKS][8];
    float gn = 0.f, gb = 0.f;
    #pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const uint2 lo = *reinterpret_cast<const uint2*>(qrow + 16 * t + 4 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(qrow + 16 * t + 8 + 4 * g);
      const uint32_t w4[4] = {lo.x, lo.y, hi.x, hi.y};
      #pragma unroll
      for (int u = 0; u < 4; ++u) {
        qop[t][2 * u] = static_cast<_Float16>(qvalid ? bf16_to_f(w4[u] & 0xffffu) * qsc : 0.f);
        qop[t][2 * u + 1] = static_cast<_Float16>(qvalid ? bf16_to_f(w4[u] >> 16) * qsc : 0.f);
      }
      const float4 g0 = *reinterpret_cast<const float4*>(grow + 16 * t + 4 * g);
      const float4 g1 = *reinterpret_cast<const float4*>(grow + 16 * t + 8 + 4 * g);
      const float4 b0 = *reinterpret_cast<const float4*>(brow + 16 * t + 4 * g);
      const float4 b1 = *reinterpret_cast<const float4*>(brow + 16 * t + 8 + 4 * g);
      const float ge[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float be[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      #pragma unroll
      for (int c = 0; c < 8; ++c) {
        gv[t][c] = qvalid ? ge[c] : 0.f;
        gn += gv[t][c] * gv[t][c];
        gb += gv[t][c] * (qvalid ? be[c] : 0.f);
      }
    }
    gn = pair_sum(gn);
    gb = pair_sum(gb);
    // |s_g g| in (32, 64]: |G| <= 2 * 64 * 128 stays far inside fp16
    sg = gn > 0.f ? pow2_floor(64.f / sqrtf(gn)) : 1.f;
    #pragma unroll
    for (int t = 0; t < NKS; ++t)
      #pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float x = gv[t][c] * sg;
        gop[t][c] = static_cast<_Float16>(x);
        glo[t][c] = static_cast<_Float16>(x - static_cast<float>(gop[t][c]));
      }
    sinit_v = -qst[lane];
    om = qst[64 + lane];
    ginit_v = -sg * sv * gb;
    gb_row = gb;
  } else {
    // from the query tile's record (written by bwd_rows); a wave past the end
    // of the head has none and takes no part in the products
    if (wave_any) {
      const char* rec = P.rec + (static_cast<size_t>(bh) * P.nblk + (wfirst >> 5)) * rec_bytes<D>();
      const float* cst = reinterpret_cast<const float*>(rec + cst_off<D>());
      auto rfrag = [&](int X, int t) __attribute__((always_inline)) {
        return *reinterpret_cast<const half8*>(rec + X * tile_bytes<D>() + (((2 * t + g) * BK + ql) * 8) * 2);
      };
      #pragma unroll
      for (int t = 0; t < NKS; ++t) {
        qop[t] = rfrag(T_QR, t);
        rh[t] = rfrag(T_RH, t);
        rl[t] = rfrag(T_RL, t);
        yop[t] = rfrag(T_YH, t);
        gop[t] = rfrag(T_GH, t);
        glo[t] = rfrag(T_GL, t);
      }
      sinit_v = cst[C_SINIT * 32 + ql];
      c_rinit = cst[C_RINIT * 32 + ql];
      c_rslope = cst[C_RSLOPE * 32 + ql];
      c_yinit = cst[C_YINIT * 32 + ql];
      ginit_v = cst[C_GINIT * 32 + ql];
      c_eg = cst[C_EG * 32 + ql];
      c_ey = cst[C_EY * 32 + ql];
      c_tau = cst[C_TAU * 32 + ql];
      jst = __float_as_int(cst[C_JSTAR * 32 + ql]);
      c_f = cst[C_F * 32 + ql];
      c_oms = cst[C_OMS * 32 + ql];
      c_dqs = cst[C_DQS * 32 + ql];
    } else {
      #pragma unroll
      for (int t = 0; t < NKS; ++t)
        #pragma unroll
        for (int c = 0; c < 8; ++c) {
          qop[t][c] = rh[t][c] = rl[t][c] = yop[t][c] = gop[t][c] = glo[t][c] = static_cast<_Float16>(0.f);
        }
    }
  }

  floatx16 acc[NMB];
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  float usum = 0.f;
  // (right-hand side) the row sums of w and of w (G - g.out): g . vbar from
  // this sweep's own weights. Through the forward's output instead, its error
  // (small against out, not against the O(lambda) residuals e_j of a nearly
  // interpolating fit, which it shifts) would reach dk multiplied by 1/lambda.
  float wsum = 0.f, wgsum = 0.f;
  float bestv = -INFINITY;
  int bestk = qvalid ? qi : 0;  // (stays a visible key even for NaN scores)

  auto copy_tile = [&](int j, int b) __attribute__((always_inline)) {
    load_kr_to_lds<D, NW>(kr_head, j, sKr[b], wave, lane);
    load_kr_to_lds<D, NW>(vr_head, j, sVr[b], wave, lane);
    load_kr_to_lds<D, NW>(kt_head, j, sKt[b], wave, lane);
  };
  // Two-stage pipeline over the key tiles: step j issues the score products
  // of tile j + 1 (into the other accumulator set), then the vector work of
  // tile j, which does not depend on them and runs while they execute, then
  // tile j's products into acc. Tile t sits in buffer t % NB: in step j the
  // waves read tiles j and j + 1 while tile j + 2 is copied into the buffer
  // of tile j - 1.
  // X[0] = S (scores, log2 units, less the row max), X[1] = G, X[2] = R, X[3] = Yp
  auto front = [&](int j, floatx16 (&X)[4]) __attribute__((always_inline)) {
    const _Float16* kb_ = sKr[j % NB];
    const _Float16* vb_ = sVr[j % NB];
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      X[0][r] = sinit_v;
      X[1][r] = ginit_v;
      X[2][r] = c_rinit;
      X[3][r] = c_yinit;
    }
    // (consecutive products write different accumulators: a dependent
    // matrix instruction would wait for its predecessor's result)
    #pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const half8 kf = kr_frag_at(kb_, t);
      const half8 vf = kr_frag_at(vb_, t);
      X[0] = mfma(kf, qop[t], X[0]);
      X[1] = mfma(vf, gop[t], X[1]);
      if constexpr (MODE == 1) {
        X[2] = mfma(kf, rh[t], X[2]);
        X[3] = mfma(kf, yop[t], X[3]);
        X[1] = mfma(vf, glo[t], X[1]);
        X[2] = mfma(kf, rl[t], X[2]);
      } else {
        X[1] = mfma(vf, glo[t], X[1]);
      }
    }
  };
  auto back = [&](int j, const floatx16 (&X)[4]) __attribute__((always_inline)) {
    const _Float16* tb_ = sKt[j % NB];
    const bool diag = (j == wlast);
    const int lim = qi - j * BK;  // keys <= lim are visible
    half8 U[2], Ul[2];
    float wv[16];
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key_of(r);
      const bool vis = qvalid && (!diag || key <= lim);
      const float x = X[0][r];
      const float w = vis ? fast_exp2(x) : 0.f;
      if constexpr (MODE == 0) {
        const int kj = j * BK + key;
        if (vis && (x > bestv || (x == bestv && kj < bestk))) {
          bestv = x;
          bestk = kj;
        }
        wv[r] = w;
        wsum += w;
        wgsum = fmaf(w, X[1][r], wgsum);
        if (r & 1) {
          // U in two fp16 terms (hi + lo): h feeds e_j = beta_j / omega -
          // c_j . y, a difference of O(1) terms that is O(lambda) where the
          // fit nearly interpolates
          const float u0 = wv[r - 1] * X[1][r - 1], u1 = w * X[1][r];
          const half2v hu = pack_sum(u0, u1, usum);
          const half2v lo = pack_sum(u0 - static_cast<float>(hu[0]), u1 - static_cast<float>(hu[1]), usum);
          U[r >> 3][(r - 1) & 7] = hu[0];
          U[r >> 3][r & 7] = hu[1];
          Ul[r >> 3][(r - 1) & 7] = lo[0];
          Ul[r >> 3][r & 7] = lo[1];
        }
      } else {
        const float A = fmaf(c_rslope, X[2][r], 1.f);
        const float e = fmaf(X[1][r], c_eg, X[3][r] * c_ey);
        wv[r] = w * fmaf(A, e, c_tau) * c_f;
        if (r & 1) {
          const half2v hu = pack_sum(wv[r - 1], wv[r], usum);
          U[r >> 3][(r - 1) & 7] = hu[0];
          U[r >> 3][r & 7] = hu[1];
        }
      }
    }
    #pragma unroll
    for (int h = 0; h < 2; ++h)
      #pragma unroll
      for (int mb = 0; mb < NMB; ++mb) acc[mb] = mfma(kt_frag_at(tb_, mb, h), U[h], acc[mb]);
    if constexpr (MODE == 0)
      #pragma unroll
      for (int h = 0; h < 2; ++h)
        #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[mb] = mfma(kt_frag_at(tb_, mb, h), Ul[h], acc[mb]);
  };
  // step j: tile j + 1 has landed everywhere (the only copy in flight), tile
  // j - 1 is no longer read; start copying tile j + 2
  auto step = [&](int j, const floatx16 (&Xc)[4], floatx16 (&Xn)[4]) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + 2 < ntiles) copy_tile(j + 2, (j + 2) % NB);
    if (j + 1 < ntiles && j + 1 <= wlast) front(j + 1, Xn);
    if (j <= wlast) back(j, Xc);
  };
  floatx16 XA[4];
  if constexpr (PIPE) {
    floatx16 XB[4];
    copy_tile(0, 0);
    if (ntiles > 1) copy_tile(1, 1);
    // tile 0 has landed (tile 1 may be in flight)
    if constexpr (NCPT == 6)
      asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (0 <= wlast) front(0, XA);
    for (int j = 0; j < ntiles; j += 2) {
      step(j, XA, XB);
      if (j + 1 < ntiles) step(j + 1, XB, XA);
    }
  } else {
    copy_tile(0, 0);
    for (int j = 0; j < ntiles; ++j) {
      // tile j has landed everywhere and tile j - 1 is no longer read
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (j + 1 < ntiles) copy_tile(j + 1, (j + 1) % NB);
      if (j > wlast) continue;
      front(j, XA);
      back(j, XA);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no tile copy in flight at exit

  if constexpr (MODE == 0) {
    usum = pair_sum(usum);
    {
      // the pair's argmax: larger score, then smaller key index
      const auto rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(bestv), __float_as_uint(bestv), false, false);
      const auto rk = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(bestk), static_cast<uint32_t>(bestk), false, false);
      const float v0 = __uint_as_float(rv[0]), v1 = __uint_as_float(rv[1]);
      const int k0 = static_cast<int>(rk[0]), k1 = static_cast<int>(rk[1]);
      const bool one = v1 > v0 || (v1 == v0 && k1 < k0);
      bestk = one ? k1 : k0;
    }
    // s h = (Y - (sum U) kbar_s) / (s_g s_v omega): the CG kernel solves
    // s^2 Sigma_c x = s h, so x = y / s
    const float inv = qvalid ? 1.f / (sg * sv * om) : 0.f;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 kb = slab_ld(kbs, mb * 4 + a, lane);
        floatx4 rc;
        #pragma unroll
        for (int b = 0; b < 4; ++b) rc[b] = (acc[mb][4 * a + b] - usum * kb[b]) * inv;
        slab_st(rsl, mb * 4 + a, lane, rc);
      }
    // g . vbar = g . out + sum_j w_j (g . v_j - g . out) / sum_j w_j
    wsum = pair_sum(wsum);
    wgsum = pair_sum(wgsum);
    if (qvalid && g == 0) {
      P.jstar[orow] = bestk;
      P.gvb[orow] = gb_row + (wsum > 0.f ? wgsum / (wsum * sg * sv) : 0.f);
    }
  } else {
    // The max's share: the row's sum of the operands the products used, taken
    // off at the maximising key, so that dq's row of dL/ds sums to zero as it
    // must whatever the rounding of its terms. (The key-major kernel takes
    // the closed form -lambda y.rho_c instead: there the share is a single
    // term, and a sum of rounded terms that nearly cancel is not accurate.)
    usum = pair_sum(usum);
    if (!qvalid) return;
    const uint16_t* kst = P.k + (static_cast<size_t>(bh) * n + min(max(jst, 0), qi)) * D;
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 y4 = slab_ld(xs, mb * 4 + a, lane);
        const uint2 k2 = *reinterpret_cast<const uint2*>(kst + 32 * mb + 8 * a + 4 * g);
        const float ke[4] = {bf16_to_f(k2.x & 0xffffu) * s, bf16_to_f(k2.x >> 16) * s,
                             bf16_to_f(k2.y & 0xffffu) * s, bf16_to_f(k2.y >> 16) * s};
        float o[4];
        #pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = fmaf(acc[mb][4 * a + b] - usum * ke[b], c_dqs, c_oms * y4[b]);
        *reinterpret_cast<float4*>(P.dq + orow * D + 32 * mb + 8 * a + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
      }
  }
}

// ---------------------------------------------------------------------------
struct RowsParams {
  const uint16_t* q;
  const float* dout;
  const float* rho_c;
  const float* partial;
  const float* xs;
  const float* kbs;
  const float* rs;
  const float* qs;
  const int32_t* jstar;
  const float* gvb;
  char* rec;
  int BH, n, nchunk, nblk, nq32;
  float lambda;
};

// Per query, after the adjoint solve: the constants of the two gradient
// sweeps and the query-tile operands. One wave
// per 32-query tile (query along lanes, as in the forward); each tile is
// assembled in LDS and written out with 16-byte stores.
template <int D>
__global__ __launch_bounds__(NT) void bwd_rows(RowsParams P) {
  constexpr int NMB = D / 32, NW = NT / 64;
  __shared__ __align__(16) uint16_t sT[NW][BK * D];
  __shared__ float sScale[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;
  const int n = P.n;
  const int nqb = (n + 32 * NW - 1) / (32 * NW);
  const int bh = static_cast<int>(blockIdx.x) / nqb, qblk = static_cast<int>(blockIdx.x) % nqb;
  const int T = qblk * NW + wave;  // this wave's 32-query tile
  const bool tvalid = T < P.nblk;
  const int qi = 32 * T + ql;
  const bool qvalid = qi < n;
  if (tid < 64) {
    float a, b, mk, mv, mq;
    head_scales(P.partial, bh, P.nchunk, tid, &a, &b);
    head_maxima(P.partial, bh, P.nchunk, tid, &mk, &mv, &mq);
    if (tid == 0) {
      sScale[0] = a;
      sScale[1] = b;
      sScale[2] = fmaxf(mk, mq);  // largest row norm of q and k together
      sScale[3] = mv;             // and of v
    }
  }
  __syncthreads();
  const float s = sScale[0], sv = sScale[1], kmax = sScale[2], vmax = sScale[3];
  const float inv_s = 1.f / s;
  const size_t wslot = static_cast<size_t>(bh) * P.nq32 + (tvalid ? T : 0);
  const __amdgpu_buffer_rsrc_t xs = make_rsrc(P.xs + wslot * (32 * D), 32 * D * 4);
  const __amdgpu_buffer_rsrc_t kbs = make_rsrc(P.kbs + wslot * (32 * D), 32 * D * 4);
  const __amdgpu_buffer_rsrc_t rsl = make_rsrc(P.rs + wslot * (32 * D), 32 * D * 4);
  const float* qst = P.qs + wslot * 128;
  const size_t orow = static_cast<size_t>(bh) * n + (qvalid ? qi : 0);

  // per-query vectors in the accumulator layout: slot (mb, a, b) is dim
  // 32 mb + 8 a + 4 g + b
  float qv[NMB][4][4], rv[NMB][4][4], gv[NMB][4][4], kb[NMB][4][4], ys[NMB][4][4];
  float gn = 0.f;
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dim = 32 * mb + 8 * a + 4 * g;
      const uint2 q2 = *reinterpret_cast<const uint2*>(P.q + orow * D + dim);
      const float4 r4 = *reinterpret_cast<const float4*>(P.rho_c + orow * D + dim);
      const float4 g4 = *reinterpret_cast<const float4*>(P.dout + orow * D + dim);
      const floatx4 k4 = tvalid ? slab_ld(kbs, mb * 4 + a, lane) : floatx4{0.f, 0.f, 0.f, 0.f};
      const floatx4 y4 = tvalid ? slab_ld(xs, mb * 4 + a, lane) : floatx4{0.f, 0.f, 0.f, 0.f};
      const float qe[4] = {bf16_to_f(q2.x & 0xffffu), bf16_to_f(q2.x >> 16), bf16_to_f(q2.y & 0xffffu),
                           bf16_to_f(q2.y >> 16)};
      const float re[4] = {r4.x, r4.y, r4.z, r4.w}, ge[4] = {g4.x, g4.y, g4.z, g4.w};
      #pragma unroll
      for (int b = 0; b < 4; ++b) {
        qv[mb][a][b] = qvalid ? qe[b] : 0.f;
        rv[mb][a][b] = qvalid ? re[b] : 0.f;
        gv[mb][a][b] = qvalid ? ge[b] : 0.f;
        kb[mb][a][b] = qvalid ? k4[b] : 0.f;
        ys[mb][a][b] = qvalid ? y4[b] : 0.f;
        gn += gv[mb][a][b] * gv[mb][a][b];
      }
    }
  gn = pair_sum(gn);
  const float sg = gn > 0.f ? pow2_floor(64.f / sqrtf(gn)) : 1.f;
  // x_s = rho_c / s is the forward's scaled iterate
  float kbx = 0.f, kby = 0.f, kap = 0.f, yu = 0.f, yx = 0.f, rn = 0.f, yn = 0.f, mxx = 0.f, mxy = 0.f;
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int a = 0; a < 4; ++a) {
      const floatx4 h4 = tvalid ? slab_ld(rsl, mb * 4 + a, lane) : floatx4{0.f, 0.f, 0.f, 0.f};
      #pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float rc = rv[mb][a][b];  // rho_c
        const float x = rc * inv_s;     // x_s
        const float y = ys[mb][a][b];
        kbx += kb[mb][a][b] * x;
        kby += kb[mb][a][b] * y;
        kap += (qvalid ? h4[b] : 0.f) * x;
        yu += y * (kb[mb][a][b] - s * qv[mb][a][b]);
        yx += y * x;
        rn += rc * rc;
        yn += y * y;
        mxx = fmaxf(mxx, fabsf(x));
        mxy = fmaxf(mxy, fabsf(y));
      }
    }
  kbx = pair_sum(kbx);
  kby = pair_sum(kby);
  kap = pair_sum(kap);
  yu = pair_sum(yu);
  yx = pair_sum(yx);
  rn = pair_sum(rn);
  yn = pair_sum(yn) * s * s;
  const float srho = pow2_ceil(pair_max(mxx));
  const float sy = pow2_ceil(pair_max(mxy));
  const float om = qst[64 + lane], m2 = qst[lane];
  const float tau = qvalid ? kap / om - yu : 0.f;
  const float msum = -scaled_ridge(P.lambda, s) * yx;
  // g . vbar, formed by the right-hand-side sweep from its weights
  const float gvbar = qvalid ? P.gvb[orow] : 0.f;
  // |dL/ds| <= (1 + 2 kmax |rho_c|)(2 |g| vmax / omega + 2 kmax |y|) + |tau|
  // (+ |msum| at the maximising key): the dq product's operand scale
  float bound = (1.f + 2.f * kmax * sqrtf(rn)) * (2.f * sqrtf(gn) * vmax / om + 2.f * kmax * sqrtf(yn)) +
                fabsf(tau) + fabsf(msum);
  const float f = (qvalid && bound > 0.f && bound < INFINITY) ? pow2_floor(8192.f / bound) : 1.f;

  if (!tvalid) return;  // (after the only block-wide barrier)
  char* rec = P.rec + (static_cast<size_t>(bh) * P.nblk + T) * rec_bytes<D>();
  {
    float* cst = reinterpret_cast<float*>(rec + cst_off<D>());
    const float inv_srho = 1.f / srho, inv_sy = 1.f / sy;
    float cv[kNConst];
    #pragma unroll
    for (int k = 0; k < kNConst; ++k) cv[k] = 0.f;
    if (qvalid) {
      cv[C_SINIT] = -m2;
      cv[C_RINIT] = -kbx * inv_srho;
      cv[C_RSLOPE] = -srho;
      cv[C_YINIT] = -kby * inv_sy;
      cv[C_GINIT] = -sg * sv * gvbar;
      cv[C_EG] = 1.f / (sg * sv * om);
      cv[C_EY] = -sy;
      cv[C_TAU] = tau;
      cv[C_MSUM] = msum;
      cv[C_JSTAR] = __int_as_float(P.jstar[orow]);
      cv[C_F] = f;
      cv[C_OMS] = om * s;
      cv[C_DQS] = 1.f / (sqrtf(static_cast<float>(D)) * f * s);
    } else {
      cv[C_JSTAR] = __int_as_float(-1);
    }
    #pragma unroll
    for (int k = 0; k < kNConst / 2; ++k) cst[(8 * g + k) * 32 + ql] = cv[8 * g + k];
  }
  const float qsc = kLog2e / sqrtf(static_cast<float>(D)) / s;
  uint16_t* buf = sT[wave];
  // copy the assembled tile X out of LDS (the wave's own buffer)
  // (one wave's LDS operations complete in order; the waits also keep the
  // compiler from moving LDS accesses across)
  // (X: byte offset of the tile in the record)
  auto flush = [&](size_t X) __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const uint4* src = reinterpret_cast<const uint4*>(buf);
    uint4* dst = reinterpret_cast<uint4*>(rec + X);
    #pragma unroll
    for (int i = 0; i < BK * D * 2 / 16 / 64; ++i) dst[i * 64 + lane] = src[i * 64 + lane];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // row layout: dims 32 mb + 8 a + 4 g + (0..3) sit at chunk 4 mb + 2 (a >> 1)
  // + g, positions 4 (a & 1) + (0..3) of row ql
  auto put_row = [&](auto fn) __attribute__((always_inline)) {
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int c = 4 * mb + 2 * (a >> 1) + g;
        _Float16 h4[4];
        #pragma unroll
        for (int b = 0; b < 4; ++b) h4[b] = static_cast<_Float16>(fn(mb, a, b));
        *reinterpret_cast<uint2*>(buf + (c * BK + ql) * 8 + 4 * (a & 1)) = __builtin_bit_cast(uint2, h4);
      }
  };
  // transposed layout: query row ql at chunk pos >> 3, position pos & 7 of
  // every dim's 8-element group, pos = (ql & 16) | swz16(ql & 15)
  const int tpos = (ql & 16) | swz16(ql & 15);
  auto put_t = [&](auto fn) __attribute__((always_inline)) {
    #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      #pragma unroll
      for (int a = 0; a < 4; ++a)
        #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int dim = 32 * mb + 8 * a + 4 * g + b;
          const __bf16 h = static_cast<__bf16>(fn(mb, a, b));
          buf[((tpos >> 3) * D + dim) * 8 + (tpos & 7)] = __builtin_bit_cast(uint16_t, h);
        }
  };
  const float inv_srho = 1.f / srho, inv_sy = 1.f / sy, inv_om = qvalid ? 1.f / om : 0.f;
  constexpr size_t TB = tile_bytes<D>();
  auto lo16 = [](float x) __attribute__((always_inline)) { return x - static_cast<float>(static_cast<_Float16>(x)); };
  put_row([&](int mb, int a, int b) { return qv[mb][a][b] * qsc; });
  flush(T_QR * TB);
  put_row([&](int mb, int a, int b) { return rv[mb][a][b] * inv_s * inv_srho; });
  flush(T_RH * TB);
  put_row([&](int mb, int a, int b) { return lo16(rv[mb][a][b] * inv_s * inv_srho); });
  flush(T_RL * TB);
  put_row([&](int mb, int a, int b) { return ys[mb][a][b] * inv_sy; });
  flush(T_YH * TB);
  put_row([&](int mb, int a, int b) { return lo16(ys[mb][a][b] * inv_sy); });
  flush(T_YL * TB);
  put_row([&](int mb, int a, int b) { return gv[mb][a][b] * sg; });
  flush(T_GH * TB);
  put_row([&](int mb, int a, int b) { return lo16(gv[mb][a][b] * sg); });
  flush(T_GL * TB);
  put_t([&](int mb, int a, int b) { return qv[mb][a][b]; });
  flush(row_part<D>() + T_QT * TB);
  put_t([&](int mb, int a, int b) { return ys[mb][a][b] * s; });
  flush(row_part<D>() + T_YT * TB);
  put_t([&](int mb, int a, int b) { return rv[mb][a][b]; });
  flush(row_part<D>() + T_RT * TB);
  put_t([&](int mb, int a, int b) { return -gv[mb][a][b] * inv_om; });
  flush(row_part<D>() + T_GT * TB);
}

// ---------------------------------------------------------------------------
struct KeyParams {
  const char* rec;
  const _Float16* kr;
  const _Float16* vr;
  float* dk;
  float* dv;
  int BH, n, nblk;
};

// Key-major sweep: each workgroup owns 128 keys (four waves of 32, the key
// along lanes) and streams the records of the query tiles at or after them.
// The row tiles and constants (read by the score products, first) are
// double-buffered; the transposed tiles (read by the output products, last)
// have one buffer, refilled once every wave is done with it. Per query tile:
//   wait for its rows (its transposed tiles may still be in flight); barrier;
//   start copying the next tile's rows; score products and vector work;
//   wait for its transposed tiles; barrier; output products; barrier; start
//   copying the next tile's transposed tiles.
template <int D>
__global__ __launch_bounds__(NT) void bwd_keys(KeyParams P) {
  constexpr int NKS = D / 16, NMB = D / 32, NW = NT / 64;
  constexpr size_t TB = tile_bytes<D>(), RP = row_part<D>(), RB = rec_bytes<D>();
  constexpr int PWR = static_cast<int>(RP / 1024) / NW;                 // row copies per wave
  constexpr int PWT = static_cast<int>(kNTransTiles * TB / 1024) / NW;  // transposed copies per wave
  static_assert(PWR <= 63 && PWT <= 63, "vmcnt range");
  __shared__ __align__(16) char sR[2][RP];
  __shared__ __align__(16) char sT[kNTransTiles * TB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;
  const int n = P.n;
  const int nkb = (n + 32 * NW - 1) / (32 * NW);
  int qb, bh;
  block_coords(static_cast<int>(blockIdx.x), P.BH, nkb, &qb, &bh, false);
  const int kb = nkb - 1 - qb;  // longest query range first
  const int KT = kb * NW + wave; // this wave's key tile
  const int kj = 32 * KT + ql;
  const bool wave_any = 32 * KT < n;
  const bool kvalid = kj < n;
  const int T0 = kb * NW;
  const float c = 1.f / sqrtf(static_cast<float>(D));

  half8 kop[NKS], vop[NKS];
  {
    const size_t tb = (static_cast<size_t>(bh) * P.nblk + (wave_any ? KT : 0)) * BK * D;
    #pragma unroll
    for (int t = 0; t < NKS; ++t) {
      kop[t] = *reinterpret_cast<const half8*>(P.kr + tb + ((2 * t + g) * BK + ql) * 8);
      vop[t] = *reinterpret_cast<const half8*>(P.vr + tb + ((2 * t + g) * BK + ql) * 8);
    }
  }
  floatx16 dk[NMB], dv[NMB];
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int r = 0; r < 16; ++r) dk[mb][r] = dv[mb][r] = 0.f;

  const char* head_rec = P.rec + static_cast<size_t>(bh) * P.nblk * RB;
  // copy `per` 1 KiB pieces per wave from byte `src_off` of record T to `dst`
  auto copy_part = [&](int T, size_t src_off, char* dst, int per) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(head_rec + static_cast<size_t>(T) * RB + src_off, static_cast<uint32_t>(RB - src_off));
    for (int u = 0; u < per; ++u) {
      const int inst = u * NW + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(dst + inst * 1024), 16, inst * 1024 + lane * 16, 0, 0, 0);
    }
  };
  copy_part(T0, 0, sR[0], PWR);
  copy_part(T0, RP, sT, PWT);
  for (int T = T0; T < P.nblk; ++T) {
    const int b = (T - T0) & 1;
    const bool more = T + 1 < P.nblk;
    // this tile's rows have landed (its transposed tiles may be in flight)
    if constexpr (PWT == 8)
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (more) copy_part(T + 1, 0, sR[b ^ 1], PWR);
    const bool active = wave_any && T >= KT;
    const char* rec = sR[b];
    bf16x8 p1[2], p2[2], p3[2];
    if (active) {
      const bool masked = (T == KT) || (T == P.nblk - 1);
      auto rfrag = [&](int X, int t) __attribute__((always_inline)) {
        return *reinterpret_cast<const half8*>(rec + X * TB + (((2 * t + g) * BK + ql) * 8) * 2);
      };
      const float* cst = reinterpret_cast<const float*>(rec + cst_off<D>());
      // constant k of the queries of accumulator registers 4 a .. 4 a + 3
      auto cvec = [&](int k, int a) __attribute__((always_inline)) {
        return *reinterpret_cast<const floatx4*>(cst + k * 32 + 8 * a + 4 * g);
      };
      floatx16 sacc, racc, yacc, gacc;
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 s4 = cvec(C_SINIT, a), r4 = cvec(C_RINIT, a), y4 = cvec(C_YINIT, a), g4 = cvec(C_GINIT, a);
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
          sacc[4 * a + e] = s4[e];
          racc[4 * a + e] = r4[e];
          yacc[4 * a + e] = y4[e];
          gacc[4 * a + e] = g4[e];
        }
      }
      // (consecutive products write different accumulators)
      #pragma unroll
      for (int t = 0; t < NKS; ++t) {
        sacc = mfma(rfrag(T_QR, t), kop[t], sacc);
        racc = mfma(rfrag(T_RH, t), kop[t], racc);
        yacc = mfma(rfrag(T_YH, t), kop[t], yacc);
        gacc = mfma(rfrag(T_GH, t), vop[t], gacc);
        racc = mfma(rfrag(T_RL, t), kop[t], racc);
        yacc = mfma(rfrag(T_YL, t), kop[t], yacc);
        gacc = mfma(rfrag(T_GL, t), vop[t], gacc);
      }
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const floatx4 rs4 = cvec(C_RSLOPE, a), eg4 = cvec(C_EG, a), ey4 = cvec(C_EY, a), ta4 = cvec(C_TAU, a),
                      ms4 = cvec(C_MSUM, a), js4 = cvec(C_JSTAR, a);
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * a + e;
          const int qrow = 32 * T + 8 * a + 4 * g + e;
          const bool vis = !masked || (kj <= qrow && qrow < n);
          const float w = vis ? fast_exp2(sacc[r]) : 0.f;
          const float A = fmaf(rs4[e], racc[r], 1.f);
          const float ev = fmaf(gacc[r], eg4[e], yacc[r] * ey4[e]);
          float sig = w * fmaf(A, ev, ta4[e]);
          if (vis && kj == __float_as_int(js4[e])) sig -= ms4[e];
          p1[r >> 3][r & 7] = static_cast<__bf16>(c * sig);
          p2[r >> 3][r & 7] = static_cast<__bf16>(-w * A);
          p3[r >> 3][r & 7] = static_cast<__bf16>(-w * ev);
        }
      }
    }
    // this tile's transposed tiles have landed (the next rows may be in flight)
    if (more) {
      if constexpr (PWR == 15)
        asm volatile("s_waitcnt vmcnt(15) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (active) {
      auto tfrag = [&](int X, int mb, int h) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(sT + X * TB + (((2 * h + g) * D + 32 * mb + ql) * 8) * 2);
      };
      // product-major order: consecutive products write different accumulators
      #pragma unroll
      for (int h = 0; h < 2; ++h) {
        #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) dk[mb] = mfma_bf(tfrag(T_QT, mb, h), p1[h], dk[mb]);
        #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) dv[mb] = mfma_bf(tfrag(T_GT, mb, h), p2[h], dv[mb]);
        #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) dk[mb] = mfma_bf(tfrag(T_YT, mb, h), p2[h], dk[mb]);
        #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) dk[mb] = mfma_bf(tfrag(T_RT, mb, h), p3[h], dk[mb]);
      }
    }
    // every wave is done with the transposed tiles
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (more) copy_part(T + 1, RP, sT, PWT);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no record copy in flight at exit
  if (!kvalid) return;
  const size_t orow = static_cast<size_t>(bh) * n + kj;
  #pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    #pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dim = 32 * mb + 8 * a + 4 * g;
      *reinterpret_cast<float4*>(P.dk + orow * D + dim) =
          make_float4(dk[mb][4 * a], dk[mb][4 * a + 1], dk[mb][4 * a + 2], dk[mb][4 * a + 3]);
      *reinterpret_cast<float4*>(P.dv + orow * D + dim) =
          make_float4(dv[mb][4 * a], dv[mb][4 * a + 1], dv[mb][4 * a + 2], dv[mb][4 * a + 3]);
    }
}

template <int D>
hipError_t bwd_d(const BwdParams& p, hipStream_t stream) {
  const int n = p.n;
  const int nchunk = (n + NORM_ROWS - 1) / NORM_ROWS;
  const int nblk = (n + BK - 1) / BK;
  const int nqb = (n + 127) / 128;
  const int nq32 = (n + kMaxBQ - 1) / kMaxBQ * (kMaxBQ / 32);
  FwdParams f{};
  f.q = p.q;
  f.k = p.k;
  f.v = p.v;
  f.BH = p.BH;
  f.n = n;
  f.d = D;
  f.dtype = p.dtype;
  f.lambda = p.lambda;
  f.cg_max_iters = p.cg_max_iters;
  f.cg_rel_tol = p.cg_rel_tol;
  f.cg_iters = p.adj_iters;
  f.cg_resid = p.adj_resid;
  f.flags = p.flags & (LLA_FLAG_SPLIT_U | LLA_FLAG_PRECOND | LLA_FLAG_NO_PRECOND);
  f.workspace = p.workspace;
  f.workspace_bytes = p.workspace_bytes;
  // (the weights of the moments in two fp16 terms: the right-hand side below
  // subtracts (sum U) kbar, which is exact only for the kbar of the sweep's own
  // weights, and a nearly interpolating fit multiplies the difference by
  // 1/lambda in dk)
  hipError_t e = mfma_moments(f, true, stream);
  if (e != hipSuccess) return e;
  const Workspace w = carve(p.workspace, p.BH, n, D);
  const BwdWorkspace bw = carve_bwd(p.workspace, p.BH, n, D);
  hipLaunchKernelGGL(prep_vrows<D>, dim3(p.BH, nblk), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(p.v), n, nchunk, nblk, w.partial, bw.vr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  SweepParams sp{};
  sp.q = static_cast<const uint16_t*>(p.q);
  sp.k = static_cast<const uint16_t*>(p.k);
  sp.out = p.out;
  sp.dout = p.dout;
  sp.partial = w.partial;
  sp.kr = w.kr;
  sp.kt = w.kt;
  sp.vr = bw.vr;
  sp.xs = w.xs;
  sp.kbs = w.kbs;
  sp.rs = w.rs;
  sp.qs = w.qs;
  sp.rec = bw.rec;
  sp.jstar = bw.jstar;
  sp.gvb = bw.gvb;
  sp.dq = p.dq;
  sp.BH = p.BH;
  sp.n = n;
  sp.nchunk = nchunk;
  sp.nblk = nblk;
  sp.nq32 = nq32;
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(nqb) * p.BH));
  hipLaunchKernelGGL((bwd_sweep<D, 0>), grid, dim3(NT), 0, stream, sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the adjoint solve takes the forward's policy, preconditioner included
  e = mfma_precond_build(f, stream);
  if (e != hipSuccess) return e;
  if (p.ev_main_begin) {
    e = hipEventRecord(p.ev_main_begin, stream);
    if (e != hipSuccess) return e;
  }
  e = mfma_cg(f, stream);
  if (e != hipSuccess) return e;
  if (p.ev_main_end) {
    e = hipEventRecord(p.ev_main_end, stream);
    if (e != hipSuccess) return e;
  }
  RowsParams rp{};
  rp.q = sp.q;
  rp.dout = p.dout;
  rp.rho_c = p.rho_c;
  rp.partial = w.partial;
  rp.xs = w.xs;
  rp.kbs = w.kbs;
  rp.rs = w.rs;
  rp.qs = w.qs;
  rp.jstar = bw.jstar;
  rp.gvb = bw.gvb;
  rp.rec = bw.rec;
  rp.BH = p.BH;
  rp.n = n;
  rp.nchunk = nchunk;
  rp.nblk = nblk;
  rp.nq32 = nq32;
  rp.lambda = p.lambda;
  hipLaunchKernelGGL(bwd_rows<D>, grid, dim3(NT), 0, stream, rp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_sweep<D, 1>), grid, dim3(NT), 0, stream, sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  KeyParams kp{};
  kp.rec = bw.rec;
  kp.kr = w.kr;
  kp.vr = bw.vr;
  kp.dk = p.dk;
  kp.dv = p.dv;
  kp.BH = p.BH;
  kp.n = n;
  kp.nblk = nblk;
  hipLaunchKernelGGL(bwd_keys<D>, grid, dim3(NT), 0, stream, kp);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int BH, int n, int d) {
  const size_t nblk = static_cast<size_t>((n + BK - 1) / BK);
  return mfma_workspace_bytes(BH, n, d) +
         align256(static_cast<size_t>(BH) * nblk * BK * d * sizeof(_Float16)) +
         align256(static_cast<size_t>(BH) * nblk * rec_bytes_d(d)) +
         align256(static_cast<size_t>(BH) * n * sizeof(int32_t)) +
         align256(static_cast<size_t>(BH) * n * sizeof(float));
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.n > kMfmaMaxN || p.BH > 0x7fffffff) return hipErrorInvalidValue;
  if (p.d == 128) return bwd_d<128>(p, stream);
  if (p.d == 64) return bwd_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lla
