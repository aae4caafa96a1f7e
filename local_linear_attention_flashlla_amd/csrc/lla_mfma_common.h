// Device helpers, constants and the workspace layout shared by the fp16
// matrix-core kernels of the forward pass and of its gradient (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

namespace lla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNW13 = 4;    // waves per workgroup of the moment and output kernels
constexpr int kNW2 = 4;     // waves per workgroup of the CG kernel
constexpr int kMaxBQ = 32 * (kNW13 > kNW2 ? kNW13 : kNW2);  // slab padding of the query axis
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

// fp16(a0 b0), fp16(a1 b1) packed, their rounded values added to acc as in
// pack_sum. v_fma_mixlo/mixhi_f16 form the fp32 product and round it to fp16
// in one instruction each (the same rounding as a multiply then a convert).
__device__ __forceinline__ half2v mul_pack_sum(float a0, float b0, float a1, float b1, float& acc) {
  uint32_t u;
  asm volatile("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(u) : "v"(a0), "v"(b0));
  asm volatile("v_fma_mixhi_f16 %0, %1, %2, 0" : "+v"(u) : "v"(a1), "v"(b1));
  const half2v h = __builtin_bit_cast(half2v, u);
  const half2v one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  acc = __builtin_amdgcn_fdot2(h, one, acc, false);
  return h;
}

// The two lanes l and l ^ 32 of a query combine their halves with one
// v_permlane32_swap (no LDS round trip): it returns the lower half of v in
// both halves of r[0] and the upper half in both halves of r[1].
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum over the 64 lanes, the result in every lane: DPP quad permutations
// and row mirrors within 16-lane rows, then v_permlane16_swap and
// v_permlane32_swap across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Prefix-Gram preconditioner of the CG solve. Queries are grouped in 32s;
// group g >= 1 is preconditioned with the scatter matrix of the first 32 g'
// keys plus the ridge, where g' = g for g < 8 and, beyond, g rounded down to
// a multiple of 2^(floor(log2 g) - 2): four prefix lengths per doubling of g,
// each built once per head ("slot") and shared by the groups up to the next.
// Group 0 is not preconditioned.
__host__ __device__ inline int pc_slot_of_group(int g) {  // g >= 1
  if (g < 8) return g - 1;
  const int e = 31 - __builtin_clz(static_cast<unsigned>(g));
  return 7 + 4 * (e - 3) + ((g >> (e - 2)) - 4);
}
__host__ __device__ inline int pc_group_of_slot(int slot) {  // g' of the slot
  if (slot < 7) return slot + 1;
  const int e = 3 + (slot - 7) / 4, q = (slot - 7) % 4;
  return (4 + q) << (e - 2);
}
// The first kWoodGroups groups of 32 queries (rows below 256) precondition
// each row with its whole prefix: the group's matrix (the scatter of the
// first 32 g keys, lam I for g = 0) and a rank-r correction by the group's own
// keys, applied per query in the CG kernel (pc_wood). A group's record, in
// halfs: U = the group's 32 keys less the group's point, two fp16 terms in
// the row-tile layout of kr (2 x 32 D); V = L^{-1} for A = I + U^T M U = L L^T
// and its transpose, two terms each in MFMA operand order (4 x 2 x 64 x 8);
// -M U in operand order, two terms (2 x 32 D).
constexpr int kWoodGroups = 8;
__host__ __device__ constexpr int wood_rec_halfs(int d) { return 128 * d + 4096; }

inline int pc_nslots(int n) {
  const int G = (n + 31) / 32;
  return G >= 2 ? pc_slot_of_group(G - 1) + 1 : 0;
}

struct Workspace {
  float* partial;   // [BH][nchunk][3]: largest row norm of k, of v, of q
  _Float16* kr;     // [BH][npad][D]      s k, d index permuted by swz16
  _Float16* kt;     // [BH][npad/32][D][32] s k transposed, key index permuted
  _Float16* vt;     // [BH][npad/32][D][32] sv v transposed, key index permuted
  float* xs;        // CG iterates: per workgroup BQ x D fp32, lane-contiguous
  float* kbs;       // fp32 kbar, same layout
  float* rs;        // CG residuals, same layout
  float* qs;        // per query row max and omega: [blocks][4 waves][2][64 lanes]
  _Float16* pcm;    // [BH][nslots][2][D*D] preconditioners M / sM, hi and lo fp16 terms,
                    // each in MFMA operand order (see pc_invert)
                    // (while they are built: the slots' fp32 Gram matrices, D x D)
  float* pcs;       // [BH][nslots] their power-of-two scales sM (0: not built)
  float* pct;       // [BH][nslots][D] key sums of the slots' prefixes (build only)
  _Float16* kb16;   // fp16 kbar for the preconditioned CG: per 32-query group, the D / 8
                    // fragments of 8 halfs in MFMA operand order, lane-contiguous (16 B per lane)
  _Float16* pcw;    // [BH][kWoodGroups] records of the rank-r corrections of the first groups'
                    // preconditioners (see pc_wood), kWoodRec<D> halfs each
  float* pcws;      // [BH][kWoodGroups][4] their scales (U, V, M U) and a valid flag
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Workspace carve(void* base, int BH, int n, int d) {
  const int nchunk = (n + NORM_ROWS - 1) / NORM_ROWS;
  const size_t npad = static_cast<size_t>((n + BK - 1) / BK) * BK;
  char* p = static_cast<char*>(base);
  Workspace w;
  w.partial = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(BH) * nchunk * 3 * sizeof(float));
  const size_t t = align256(static_cast<size_t>(BH) * npad * d * sizeof(_Float16));
  w.kr = reinterpret_cast<_Float16*>(p);
  p += t;
  w.kt = reinterpret_cast<_Float16*>(p);
  p += t;
  w.vt = reinterpret_cast<_Float16*>(p);
  p += t;
  const size_t nqpad = static_cast<size_t>((n + kMaxBQ - 1) / kMaxBQ) * kMaxBQ;
  const size_t sl = align256(static_cast<size_t>(BH) * nqpad * d * sizeof(float));
  w.xs = reinterpret_cast<float*>(p);
  p += sl;
  w.kbs = reinterpret_cast<float*>(p);
  p += sl;
  w.rs = reinterpret_cast<float*>(p);
  p += sl;
  w.qs = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(BH) * nqpad * 4 * sizeof(float));
  const size_t nsl = static_cast<size_t>(pc_nslots(n));
  w.pcm = reinterpret_cast<_Float16*>(p);
  p += align256(static_cast<size_t>(BH) * nsl * 2 * d * d * sizeof(_Float16));
  w.pcs = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(BH) * nsl * sizeof(float));
  w.pct = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(BH) * nsl * d * sizeof(float));
  w.kb16 = reinterpret_cast<_Float16*>(p);
  p += align256(static_cast<size_t>(BH) * nqpad * d * sizeof(_Float16));
  w.pcw = reinterpret_cast<_Float16*>(p);
  p += align256(static_cast<size_t>(BH) * kWoodGroups * wood_rec_halfs(d) * sizeof(_Float16));
  w.pcws = reinterpret_cast<float*>(p);
  return w;
}

// Largest row norms of one head (of k, of v and of q) from its chunk
// partials. Called by every lane of one wave: each lane takes every 64th
// chunk, then a 64-lane maximum; every lane gets the results.
__device__ __forceinline__ void head_maxima(const float* partial, int bh, int nchunk, int lane,
                                            float* mk, float* mv, float* mq) {
  float a = 0.f, b = 0.f, c = 0.f;
  for (int ch = lane; ch < nchunk; ch += 64) {
    const float* pr = partial + (static_cast<size_t>(bh) * nchunk + ch) * 3;
    a = fmaxf(a, pr[0]);
    b = fmaxf(b, pr[1]);
    c = fmaxf(c, pr[2]);
  }
  *mk = wave_max(a);
  *mv = wave_max(b);
  *mq = wave_max(c);
}

// Per-head power-of-two scales s (keys) and sv (values) that bring the
// largest key row norm and the largest value row norm to (64, 128]. The keys
// alone set s: the fit's geometry lives in the keys, which then keep fp16's
// full precision down to rows about 2^-17 of the largest. Queries enter the
// matrix products only as q log2(e) / (sqrt(d) s), whose fp16 rounding error
// is absolute and meets keys of norm at most 128, so small query rows cost
// nothing; the operand overflows fp16 only when a query and a key row norm
// multiply to more than about 2^25 (scores beyond a million nats). Called
// by every lane of one wave.
__device__ __forceinline__ void head_scales(const float* partial, int bh, int nchunk, int lane,
                                            float* s, float* sv) {
  float a, b, mq;
  head_maxima(partial, bh, nchunk, lane, &a, &b, &mq);
  // bounds: any bf16 value row fits (sv only ever divides out); s stays
  // where 1 / s and s^2-scaled sums are finite fp32
  *s = a > 0.f ? fminf(fmaxf(pow2_floor(kRowNormCap / a), 0x1p-100f), 0x1p100f) : 1.f;
  *sv = b > 0.f ? fminf(fmaxf(pow2_floor(kRowNormCap / b), 0x1p-120f), 0x1p120f) : 1.f;
}

// The ridge in key-scaled units, lambda s^2, held below 2^100: keys scaled to
// norms of at most 128 make the fit's own terms tiny next to that, so
// clamping changes rho by far less than fp32 resolves (rho ~ 0 either way)
// while an infinite ridge would turn the CG step into 0 * inf.
__device__ __forceinline__ float scaled_ridge(float lambda, float s) {
  return fminf(lambda * s * s, 0x1p100f);
}

// Buffer resource over `bytes` bytes at `base` (raw, untyped; reads past the
// end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// 16-byte chunk `chunk` of lane `lane` in a lane-contiguous state slab
// ([chunk][64 lanes] x 16 bytes)
__device__ __forceinline__ floatx4 slab_ld(__amdgpu_buffer_rsrc_t r, int chunk, int lane) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, chunk * 1024, 0));
}
__device__ __forceinline__ void slab_st(__amdgpu_buffer_rsrc_t r, int chunk, int lane, floatx4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, lane * 16, chunk * 1024, 0);
}

// Copy key tile `kt` of this head (rows or transposed, both BK x D fp16,
// contiguous in global memory) into an LDS tile with global_load_lds: each
// wave instruction moves 1 KiB, lane l its l-th 16 bytes; the four waves
// together copy the tile. Completion is awaited by a later barrier.
template <int D, int NW>
__device__ __forceinline__ void load_kr_to_lds(__amdgpu_buffer_rsrc_t head, int kt, _Float16* buf,
                                               int wave, int lane) {
  constexpr int NI = D / 16;  // 1 KiB instructions per tile
  const int tile_off = kt * (BK * D * 2);  // bytes, wave-uniform
  #pragma unroll
  for (int u = 0; u < (NI + NW - 1) / NW; ++u) {
    const int inst = u * NW + wave;
    if (NI % NW == 0 || inst < NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          head, (__attribute__((address_space(3))) void*)(buf + inst * 512), 16,
          inst * 1024 + lane * 16, tile_off, 0, 0);
  }
}
// Copy instruction u (of ceil(D/16 / NW)) of this wave's share of a tile.
template <int D, int NW>
__device__ __forceinline__ void load_chunk_to_lds(__amdgpu_buffer_rsrc_t head, int kt, _Float16* buf,
                                                  int wave, int lane, int u) {
  constexpr int NI = D / 16;
  const int inst = u * NW + wave;
  if (NI % NW == 0 || inst < NI)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        head, (__attribute__((address_space(3))) void*)(buf + inst * 512), 16,
        inst * 1024 + lane * 16, kt * (BK * D * 2), 0, 0);
}
template <int D, int NW>
__device__ __forceinline__ void load_kt_to_lds(__amdgpu_buffer_rsrc_t head, int kt, _Float16* buf,
                                               int wave, int lane) {
  load_kr_to_lds<D, NW>(head, kt, buf, wave, lane);
}
template <int D, int NW>
__device__ __forceinline__ void load_tile_to_lds(__amdgpu_buffer_rsrc_t kr_head,
                                                 __amdgpu_buffer_rsrc_t t_head, int kt,
                                                 _Float16* sKr, _Float16* sKt, int wave, int lane) {
  load_kr_to_lds<D, NW>(kr_head, kt, sKr, wave, lane);
  load_kt_to_lds<D, NW>(t_head, kt, sKt, wave, lane);
}

// End of a step of a pipelined sweep: wait until at most the copies of the
// last two steps (NS tiles per step, ceil(D/16 / NW) instructions each per
// wave) are still in flight, i.e. this wave's copies of two steps ago have
// landed, and all LDS reads of this step are done; then a barrier, after
// which every wave's copies of two steps ago are visible. The asm statement
// is also a compiler memory barrier: no memory access moves across.
template <int D, int NW, int NS = 2>
__device__ __forceinline__ void step_barrier() {
  constexpr int per_step = NS * ((D / 16 + NW - 1) / NW);
  static_assert(per_step == 1 || per_step == 2 || per_step == 4, "vmcnt below");
  if constexpr (per_step == 4)
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (per_step == 2)
    asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work order. Workgroups are handed to the eight XCDs (each with its own L2)
// in turn: block b runs on XCD b % 8. The first block of every head goes
// first: its sweeps are short, but its queries (prefixes shorter than d, the
// nearly interpolating fits) can take the most CG steps, which makes it the
// latest to finish when it starts last. After those, when the head count
// divides by 8, each XCD walks its own heads one after the other, every head's
// query blocks longest causal prefix first, so the key tiles that an XCD's
// workgroups stream are those of about one head at a time and stay in its L2;
// otherwise the order is longest prefix first across all heads.
// (first_block_first = false keeps the plain order, for a kernel whose
// blocks are not query blocks.)
constexpr int kXcds = 8;
__device__ __forceinline__ void block_coords(int b, int BH, int nqb, int* qb, int* bh,
                                             bool first_block_first = true) {
  if (!first_block_first) {
    if (BH % kXcds == 0) {
      const int xcd = b % kXcds, j = b / kXcds;
      *bh = xcd * (BH / kXcds) + j / nqb;
      *qb = nqb - 1 - j % nqb;
    } else {
      *qb = nqb - 1 - b / BH;
      *bh = b % BH;
    }
    return;
  }
  if (BH % kXcds == 0) {
    const int xcd = b % kXcds, j = b / kXcds;
    const int heads_per_xcd = BH / kXcds;
    if (j < heads_per_xcd) {
      *bh = xcd * heads_per_xcd + j;
      *qb = 0;
    } else {
      const int jr = j - heads_per_xcd;  // nqb >= 2 here
      *bh = xcd * heads_per_xcd + jr / (nqb - 1);
      *qb = nqb - 1 - jr % (nqb - 1);
    }
  } else if (b < BH) {
    *qb = 0;
    *bh = b;
  } else {
    *qb = nqb - 1 - (b - BH) / BH;
    *bh = (b - BH) % BH;
  }
}
}  // namespace
}  // namespace lla
