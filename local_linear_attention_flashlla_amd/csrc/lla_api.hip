// Host side of liblla.so: argument validation, kernel dispatch, workspace
// handling and status reporting for the C ABI declared in include/lla.h.
//
// Validation is pure host arithmetic on the arguments (no device call), so a
// rejected call enqueues nothing and writes nothing.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/lla.h"
#include "lla_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) overlap (byte ranges).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool d_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Longest sequence the forward takes on the vector path (see validate). The
// matrix-core path takes n <= lla::kMfmaMaxN (its key-tile offsets are 32-bit
// byte counts formed in int arithmetic).
constexpr int kMaxForwardN = 1 << 23;

// Resolve LLA_KERNEL_AUTO and check the choice for this sequence length.
// AUTO takes the matrix cores whenever they support the call (bf16, d in
// {64, 128}, n within their limit), the vector path otherwise. Returns LLA_OK
// or a status; nothing has been enqueued or allocated at this point.
int resolve_kernel(int dtype, int d, int n, int requested, int* chosen) {
  const bool mfma_ok = lla::mfma_supported(dtype, d) && n <= lla::kMfmaMaxN;
  if (requested == LLA_KERNEL_AUTO) {
    *chosen = mfma_ok ? LLA_KERNEL_MFMA : LLA_KERNEL_VALU;
    return LLA_OK;
  }
  if (requested == LLA_KERNEL_VALU) {
    *chosen = LLA_KERNEL_VALU;
    return LLA_OK;
  }
  if (requested == LLA_KERNEL_MFMA) {
    if (!lla::mfma_supported(dtype, d))
      return fail(LLA_ERR_UNSUPPORTED, "MFMA kernel needs bf16 inputs and d in {64,128} (dtype=%d d=%d)",
                  dtype, d);
    if (n > lla::kMfmaMaxN)
      return fail(LLA_ERR_UNSUPPORTED, "MFMA kernel takes n <= 2^21 (n=%d)", n);
    *chosen = LLA_KERNEL_MFMA;
    return LLA_OK;
  }
  return fail(LLA_ERR_INVALID_ARG, "unknown kernel choice %d", requested);
}

int validate(const lla_fwd_args* a) {
  if (!a) return fail(LLA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != LLA_DTYPE_F32 && a->dtype != LLA_DTYPE_BF16)
    return fail(LLA_ERR_INVALID_ARG, "unknown dtype %d", a->dtype);
  if (!a->q || !a->k || !a->v || !a->out)
    return fail(LLA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (a->B < 1 || a->H < 1 || a->n < 1)
    return fail(LLA_ERR_INVALID_ARG, "B, H, n must be >= 1 (B=%d H=%d n=%d)", a->B, a->H, a->n);
  if (!d_supported(a->d)) return fail(LLA_ERR_UNSUPPORTED, "d=%d not in {16,32,64,128}", a->d);
  // one head's key tiles are addressed through buffer resources with a
  // 32-bit byte range: n <= 2^23 keeps them at or under 2 GiB for every d
  if (a->n > kMaxForwardN) return fail(LLA_ERR_UNSUPPORTED, "n=%d > 2^23", a->n);
  if (!std::isfinite(a->lambda) || !(a->lambda > 0.f))
    return fail(LLA_ERR_INVALID_ARG, "lambda must be finite and > 0 (got %g)", (double)a->lambda);
  if (a->cg_max_iters < 0 || a->cg_max_iters > 100000)
    return fail(LLA_ERR_INVALID_ARG, "cg_max_iters must be in [0, 100000] (got %d)", a->cg_max_iters);
  if (!(a->cg_rel_tol >= 0.f) || !std::isfinite(a->cg_rel_tol))
    return fail(LLA_ERR_INVALID_ARG, "cg_rel_tol must be finite and >= 0 (got %g)", (double)a->cg_rel_tol);
  if (a->flags & ~(LLA_FLAG_SPLIT_U | LLA_FLAG_PRECOND | LLA_FLAG_NO_PRECOND))
    return fail(LLA_ERR_INVALID_ARG, "unknown flags 0x%x", a->flags);
  if ((a->flags & LLA_FLAG_PRECOND) && (a->flags & LLA_FLAG_NO_PRECOND))
    return fail(LLA_ERR_INVALID_ARG, "LLA_FLAG_PRECOND and LLA_FLAG_NO_PRECOND together");
  // sizes: every element count must fit comfortably in 64-bit and the grid in 2^31
  const unsigned long long bh = (unsigned long long)a->B * (unsigned long long)a->H;
  if (bh > 0x7fffffffULL) return fail(LLA_ERR_UNSUPPORTED, "B*H too large");
  const unsigned long long rows = bh * (unsigned long long)a->n;
  if (rows > (1ULL << 40)) return fail(LLA_ERR_UNSUPPORTED, "B*H*n too large");
  const unsigned long long grid = bh * (unsigned long long)((a->n + 31) / 32);
  if (grid > 0x7fffffffULL) return fail(LLA_ERR_UNSUPPORTED, "grid too large");
  const size_t esz = a->dtype == LLA_DTYPE_F32 ? 4 : 2;
  const size_t nin = (size_t)(rows * (unsigned long long)a->d) * esz;
  const size_t nout = (size_t)(rows * (unsigned long long)a->d) * 4;
  const size_t nrow = (size_t)rows * 4;
  const void* ins[3] = {a->q, a->k, a->v};
  for (const void* in : ins) {
    if (!aligned16(in)) return fail(LLA_ERR_INVALID_ARG, "input pointer %p not 16-byte aligned", in);
  }
  struct Out { const void* p; size_t bytes; const char* name; };
  const Out outs[7] = {{a->out, nout, "out"},           {a->rho, nout, "rho"},
                       {a->omega, nrow, "omega"},       {a->rowmax, nrow, "rowmax"},
                       {a->cg_iters, nrow, "cg_iters"}, {a->cg_resid, nrow, "cg_resid"},
                       {a->rho_c, nout, "rho_c"}};
  for (int i = 0; i < 7; ++i) {
    if (!outs[i].p) continue;
    if (!aligned16(outs[i].p))
      return fail(LLA_ERR_INVALID_ARG, "%s pointer %p not 16-byte aligned", outs[i].name, outs[i].p);
    for (const void* in : ins)
      if (overlap(outs[i].p, outs[i].bytes, in, nin))
        return fail(LLA_ERR_INVALID_ARG, "%s overlaps an input", outs[i].name);
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
        return fail(LLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  if (a->workspace && !aligned16(a->workspace))
    return fail(LLA_ERR_INVALID_ARG, "workspace pointer not 16-byte aligned");
  return LLA_OK;
}

}  // namespace

extern "C" {

const char* lla_status_string(int status) {
  switch (status) {
    case LLA_OK: return "LLA_OK";
    case LLA_ERR_INVALID_ARG: return "LLA_ERR_INVALID_ARG";
    case LLA_ERR_UNSUPPORTED: return "LLA_ERR_UNSUPPORTED";
    case LLA_ERR_HIP: return "LLA_ERR_HIP";
    case LLA_ERR_WORKSPACE: return "LLA_ERR_WORKSPACE";
    default: return "LLA_ERR_UNKNOWN";
  }
}

const char* lla_last_error(void) { return g_last_error; }

int lla_version(void) { return LLA_VERSION; }

// The build script passes the hash of the sources and flags it compiled.
#ifndef LLA_SOURCE_SHA256
#define LLA_SOURCE_SHA256 "unknown"
#endif
const char* lla_source_hash(void) { return LLA_SOURCE_SHA256; }

size_t lla_workspace_bytes(int B, int H, int n, int d, int dtype, int kernel) {
  if (B < 1 || H < 1 || n < 1 || n > kMaxForwardN || !d_supported(d)) return 0;
  if (dtype != LLA_DTYPE_F32 && dtype != LLA_DTYPE_BF16) return 0;
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 0x7fffffffULL || bh * (unsigned long long)n > (1ULL << 40)) return 0;
  int chosen = 0;
  char saved[sizeof(g_last_error)];
  memcpy(saved, g_last_error, sizeof(saved));
  const int st = resolve_kernel(dtype, d, n, kernel, &chosen);
  memcpy(g_last_error, saved, sizeof(saved));
  if (st != LLA_OK) return 0;
  if (chosen == LLA_KERNEL_MFMA) return lla::mfma_workspace_bytes(static_cast<int>(bh), n, d);
  return 0;
}

static int forward_impl(const lla_fwd_args* a, const float* rho_in, hipStream_t stream) {
  int st = validate(a);
  if (st != LLA_OK) return st;
  int kernel = 0;
  st = resolve_kernel(a->dtype, a->d, a->n, a->kernel, &kernel);
  if (st != LLA_OK) return st;
  lla::FwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out;
  p.omega = a->omega; p.rho = a->rho; p.rowmax = a->rowmax;
  p.cg_iters = a->cg_iters; p.cg_resid = a->cg_resid;
  p.rho_in = rho_in;
  p.rho_c = a->rho_c;
  p.BH = a->B * a->H; p.n = a->n; p.d = a->d; p.dtype = a->dtype;
  p.lambda = a->lambda; p.cg_max_iters = a->cg_max_iters; p.cg_rel_tol = a->cg_rel_tol;
  p.flags = a->flags;
  p.ev_main_begin = a->ev_main_begin;
  p.ev_main_end = a->ev_main_end;
  if (kernel == LLA_KERNEL_VALU) {
    const hipError_t e = lla::launch_valu(p, stream);
    if (e != hipSuccess) return fail(LLA_ERR_HIP, "VALU launch: %s", hipGetErrorString(e));
    return LLA_OK;
  }
  // MFMA: needs a workspace
  const size_t need = lla::mfma_workspace_bytes(p.BH, p.n, p.d);
  void* ws = a->workspace;
  bool owned = false;
  if (ws) {
    if (a->workspace_bytes < need)
      return fail(LLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", a->workspace_bytes, need);
  } else if (need > 0) {
    const hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return fail(LLA_ERR_HIP, "workspace allocation of %zu bytes: %s", need,
                                     hipGetErrorString(e));
    owned = true;
  }
  p.workspace = ws;
  p.workspace_bytes = owned ? need : a->workspace_bytes;
  const hipError_t e = lla::launch_mfma(p, stream);
  if (owned) {
    const hipError_t f = hipFreeAsync(ws, stream);
    if (e == hipSuccess && f != hipSuccess)
      return fail(LLA_ERR_HIP, "workspace free: %s", hipGetErrorString(f));
  }
  if (e != hipSuccess) return fail(LLA_ERR_HIP, "MFMA launch: %s", hipGetErrorString(e));
  return LLA_OK;
}

int lla_forward_ex(const lla_fwd_args* a, hipStream_t stream) {
  g_last_error[0] = '\0';
  return forward_impl(a, nullptr, stream);
}

int lla_output_given_rho(const lla_fwd_args* a, const float* rho_in, hipStream_t stream) {
  g_last_error[0] = '\0';
  const int st = validate(a);  // (sizes are checked before they are multiplied below)
  if (st != LLA_OK) return st;
  if (!rho_in) return fail(LLA_ERR_INVALID_ARG, "rho_in is NULL");
  if (a->rho_c) return fail(LLA_ERR_INVALID_ARG, "rho_c is not defined when rho is supplied");
  if (!aligned16(rho_in)) return fail(LLA_ERR_INVALID_ARG, "rho_in pointer not 16-byte aligned");
  {
    const size_t nrho = (size_t)a->B * a->H * a->n * a->d * sizeof(float);
    const size_t nrow = (size_t)a->B * a->H * a->n * sizeof(float);
    struct Out { const void* p; size_t bytes; const char* name; };
    const Out outs[6] = {{a->out, nrho, "out"},           {a->rho, nrho, "rho"},
                         {a->omega, nrow, "omega"},       {a->rowmax, nrow, "rowmax"},
                         {a->cg_iters, nrow, "cg_iters"}, {a->cg_resid, nrow, "cg_resid"}};
    for (const Out& o : outs)
      if (o.p && overlap(o.p, o.bytes, rho_in, nrho))
        return fail(LLA_ERR_INVALID_ARG, "%s overlaps rho_in", o.name);
  }
  return forward_impl(a, rho_in, stream);
}

// Longest sequence and most heads of the naive forward: its grid holds n
// rows in x and B*H heads in y (at most 65535), and its workspace grows as
// B*H*n^2*d.
constexpr int kMaxNaiveN = 1 << 16;

// Checks of a naive call beyond validate(): sizes, and the fields that have
// no meaning for it.
static int naive_check(const lla_fwd_args* a) {
  if (a->n > kMaxNaiveN) return fail(LLA_ERR_UNSUPPORTED, "naive forward: n=%d > 2^16", a->n);
  if ((unsigned long long)a->B * (unsigned long long)a->H > 65535ULL)
    return fail(LLA_ERR_UNSUPPORTED, "naive forward: B*H > 65535");
  if (a->kernel != LLA_KERNEL_AUTO)
    return fail(LLA_ERR_INVALID_ARG, "naive forward: kernel must be LLA_KERNEL_AUTO (got %d)", a->kernel);
  if (a->flags != 0) return fail(LLA_ERR_INVALID_ARG, "naive forward: flags must be 0 (got 0x%x)", a->flags);
  if (a->rho_c) return fail(LLA_ERR_INVALID_ARG, "naive forward: rho_c is not produced (exact solve)");
  return LLA_OK;
}

size_t lla_naive_workspace_bytes(int B, int H, int n, int d, int dtype) {
  if (B < 1 || H < 1 || n < 1 || n > kMaxNaiveN || !d_supported(d)) return 0;
  if (dtype != LLA_DTYPE_F32 && dtype != LLA_DTYPE_BF16) return 0;
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 65535ULL) return 0;
  return lla::naive_workspace_bytes(static_cast<int>(bh), n, d);
}

int lla_forward_naive(const lla_fwd_args* a, hipStream_t stream) {
  g_last_error[0] = '\0';
  int st = validate(a);
  if (st != LLA_OK) return st;
  st = naive_check(a);
  if (st != LLA_OK) return st;
  lla::FwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out;
  p.omega = a->omega; p.rho = a->rho; p.rowmax = a->rowmax;
  p.cg_iters = a->cg_iters; p.cg_resid = a->cg_resid;
  p.BH = a->B * a->H; p.n = a->n; p.d = a->d; p.dtype = a->dtype;
  p.lambda = a->lambda;
  p.ev_main_begin = a->ev_main_begin;
  p.ev_main_end = a->ev_main_end;
  const size_t need = lla::naive_workspace_bytes(p.BH, p.n, p.d);
  void* ws = a->workspace;
  bool owned = false;
  if (ws) {
    if (a->workspace_bytes < need)
      return fail(LLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", a->workspace_bytes, need);
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return fail(LLA_ERR_HIP, "workspace allocation of %zu bytes: %s", need,
                                     hipGetErrorString(e));
    owned = true;
  }
  p.workspace = ws;
  p.workspace_bytes = owned ? need : a->workspace_bytes;
  const hipError_t e = lla::launch_naive(p, stream);
  if (owned) {
    const hipError_t f = hipFreeAsync(ws, stream);
    if (e == hipSuccess && f != hipSuccess)
      return fail(LLA_ERR_HIP, "workspace free: %s", hipGetErrorString(f));
  }
  if (e != hipSuccess) return fail(LLA_ERR_HIP, "naive launch: %s", hipGetErrorString(e));
  return LLA_OK;
}

// Host checks of a decode call; fills *p (everything but the workspace).
static int decode_validate(const lla_decode_args* a, lla::DecodeParams* p) {
  if (!a) return fail(LLA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != LLA_DTYPE_F32 && a->dtype != LLA_DTYPE_BF16)
    return fail(LLA_ERR_INVALID_ARG, "unknown dtype %d", a->dtype);
  if (!a->q || !a->k || !a->v || !a->out)
    return fail(LLA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (a->B < 1 || a->H < 1 || a->n < 1)
    return fail(LLA_ERR_INVALID_ARG, "B, H, n must be >= 1 (B=%d H=%d n=%d)", a->B, a->H, a->n);
  if (!lla::decode_supported(a->d)) return fail(LLA_ERR_UNSUPPORTED, "decode: d=%d not in {64,128}", a->d);
  if (!std::isfinite(a->lambda) || !(a->lambda > 0.f))
    return fail(LLA_ERR_INVALID_ARG, "lambda must be finite and > 0 (got %g)", (double)a->lambda);
  if (a->cg_max_iters < 0 || a->cg_max_iters > 100000)
    return fail(LLA_ERR_INVALID_ARG, "cg_max_iters must be in [0, 100000] (got %d)", a->cg_max_iters);
  if (!(a->cg_rel_tol >= 0.f) || !std::isfinite(a->cg_rel_tol))
    return fail(LLA_ERR_INVALID_ARG, "cg_rel_tol must be finite and >= 0 (got %g)", (double)a->cg_rel_tol);
  const unsigned long long bh = (unsigned long long)a->B * (unsigned long long)a->H;
  if (bh > 65535ULL) return fail(LLA_ERR_UNSUPPORTED, "decode: B*H = %llu > 65535", bh);
  const unsigned long long keys = bh * (unsigned long long)a->n;
  if (keys > (1ULL << 36)) return fail(LLA_ERR_UNSUPPORTED, "B*H*n too large");
  const size_t esz = a->dtype == LLA_DTYPE_F32 ? 4 : 2;
  if ((unsigned long long)a->n * a->d * esz >= (1ULL << 31))
    return fail(LLA_ERR_UNSUPPORTED, "decode: one head's cache (n*d elements) must stay under 2 GiB");
  const size_t nq = (size_t)bh * a->d * esz, nkv = (size_t)keys * a->d * esz;
  const size_t nout = (size_t)bh * a->d * 4, nrow = (size_t)bh * 4;
  struct In { const void* p; size_t bytes; };
  const In ins[3] = {{a->q, nq}, {a->k, nkv}, {a->v, nkv}};
  for (const In& in : ins)
    if (!aligned16(in.p)) return fail(LLA_ERR_INVALID_ARG, "input pointer %p not 16-byte aligned", in.p);
  struct Out { const void* p; size_t bytes; const char* name; };
  const Out outs[6] = {{a->out, nout, "out"},           {a->rho, nout, "rho"},
                       {a->omega, nrow, "omega"},       {a->rowmax, nrow, "rowmax"},
                       {a->cg_iters, nrow, "cg_iters"}, {a->cg_resid, nrow, "cg_resid"}};
  for (int i = 0; i < 6; ++i) {
    if (!outs[i].p) continue;
    if (!aligned16(outs[i].p))
      return fail(LLA_ERR_INVALID_ARG, "%s pointer %p not 16-byte aligned", outs[i].name, outs[i].p);
    for (const In& in : ins)
      if (overlap(outs[i].p, outs[i].bytes, in.p, in.bytes))
        return fail(LLA_ERR_INVALID_ARG, "%s overlaps an input", outs[i].name);
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
        return fail(LLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  if (a->workspace && !aligned16(a->workspace))
    return fail(LLA_ERR_INVALID_ARG, "workspace pointer not 16-byte aligned");
  *p = lla::DecodeParams{};
  p->q = a->q; p->k = a->k; p->v = a->v; p->out = a->out;
  p->omega = a->omega; p->rho = a->rho; p->rowmax = a->rowmax;
  p->cg_iters = a->cg_iters; p->cg_resid = a->cg_resid;
  p->BH = (int)bh; p->n = a->n; p->d = a->d; p->dtype = a->dtype;
  p->lambda = a->lambda; p->cg_max_iters = a->cg_max_iters; p->cg_rel_tol = a->cg_rel_tol;
  p->ev_main_begin = a->ev_main_begin;
  p->ev_main_end = a->ev_main_end;
  return LLA_OK;
}

int lla_decode_ex(const lla_decode_args* a, hipStream_t stream) {
  g_last_error[0] = '\0';
  lla::DecodeParams p;
  const int st = decode_validate(a, &p);
  if (st != LLA_OK) return st;
  const size_t need = lla::decode_workspace_bytes(p.BH, p.n, p.d, p.dtype);
  void* ws = a->workspace;
  bool owned = false;
  if (ws) {
    if (a->workspace_bytes < need)
      return fail(LLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", a->workspace_bytes, need);
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return fail(LLA_ERR_HIP, "workspace allocation of %zu bytes: %s", need,
                                     hipGetErrorString(e));
    owned = true;
  }
  p.workspace = ws;
  p.workspace_bytes = owned ? need : a->workspace_bytes;
  const hipError_t e = lla::launch_decode(p, stream);
  if (owned) {
    const hipError_t f = hipFreeAsync(ws, stream);
    if (e == hipSuccess && f != hipSuccess)
      return fail(LLA_ERR_HIP, "workspace free: %s", hipGetErrorString(f));
  }
  if (e != hipSuccess) return fail(LLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return LLA_OK;
}

int lla_decode_noalloc(const lla_decode_args* a, hipStream_t stream) {
  g_last_error[0] = '\0';
  lla::DecodeParams p;
  const int st = decode_validate(a, &p);
  if (st != LLA_OK) return st;
  if (a->workspace || a->workspace_bytes)
    return fail(LLA_ERR_INVALID_ARG, "lla_decode_noalloc takes no workspace (its scratch is static)");
  const size_t need = lla::decode_workspace_bytes(p.BH, p.n, p.d, p.dtype);
  if (need > lla::kDecodeScratchBytes)
    return fail(LLA_ERR_WORKSPACE, "decode needs %zu bytes of scratch; the static scratch holds %zu "
                "(use lla_decode_ex with a workspace)", need, lla::kDecodeScratchBytes);
  // the stream must run on the current device, whose copy of the scratch is used
  if (stream) {
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(LLA_ERR_HIP, "device query: %s", hipGetErrorString(e));
    if (sdev != cur)
      return fail(LLA_ERR_INVALID_ARG, "stream belongs to device %d, the current device is %d", sdev, cur);
  }
  void* scratch = nullptr;
  hipError_t e = lla::decode_scratch(&scratch);
  if (e != hipSuccess) return fail(LLA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  p.workspace = scratch;
  p.workspace_bytes = lla::kDecodeScratchBytes;
  e = lla::launch_decode(p, stream);
  if (e != hipSuccess) return fail(LLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return LLA_OK;
}

size_t lla_decode_workspace_bytes(int B, int H, int n, int d, int dtype) {
  if (B < 1 || H < 1 || n < 1 || !lla::decode_supported(d)) return 0;
  if (dtype != LLA_DTYPE_F32 && dtype != LLA_DTYPE_BF16) return 0;
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 65535ULL || bh * (unsigned long long)n > (1ULL << 36)) return 0;
  return lla::decode_workspace_bytes((int)bh, n, d, dtype);
}

int lla_backward_ex(const lla_bwd_args* a, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!a) return fail(LLA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != LLA_DTYPE_F32 && a->dtype != LLA_DTYPE_BF16)
    return fail(LLA_ERR_INVALID_ARG, "unknown dtype %d", a->dtype);
  if (!a->q || !a->k || !a->v || !a->out || !a->dout || !a->rho_c || !a->dq || !a->dk || !a->dv)
    return fail(LLA_ERR_INVALID_ARG, "q, k, v, out, dout, rho_c, dq, dk and dv must be non-NULL");
  if (a->B < 1 || a->H < 1 || a->n < 1)
    return fail(LLA_ERR_INVALID_ARG, "B, H, n must be >= 1 (B=%d H=%d n=%d)", a->B, a->H, a->n);
  if (!d_supported(a->d)) return fail(LLA_ERR_UNSUPPORTED, "d=%d not in {16,32,64,128}", a->d);
  int kernel = 0;
  {
    const int st = resolve_kernel(a->dtype, a->d, a->n, a->kernel, &kernel);
    if (st != LLA_OK) return st;
  }
  if (!std::isfinite(a->lambda) || !(a->lambda > 0.f))
    return fail(LLA_ERR_INVALID_ARG, "lambda must be finite and > 0 (got %g)", (double)a->lambda);
  if (a->cg_max_iters < 0 || a->cg_max_iters > 100000)
    return fail(LLA_ERR_INVALID_ARG, "cg_max_iters must be in [0, 100000] (got %d)", a->cg_max_iters);
  if (!(a->cg_rel_tol >= 0.f) || !std::isfinite(a->cg_rel_tol))
    return fail(LLA_ERR_INVALID_ARG, "cg_rel_tol must be finite and >= 0 (got %g)", (double)a->cg_rel_tol);
  const unsigned long long bh = (unsigned long long)a->B * (unsigned long long)a->H;
  if (bh > 0x7fffffffULL) return fail(LLA_ERR_UNSUPPORTED, "B*H too large");
  if (a->n > lla::kMfmaMaxN) return fail(LLA_ERR_UNSUPPORTED, "backward: n=%d > 2^21", a->n);
  const unsigned long long rows = bh * (unsigned long long)a->n;
  if (rows > (1ULL << 40) || bh * (unsigned long long)((a->n + 127) / 128) > 0x7fffffffULL)
    return fail(LLA_ERR_UNSUPPORTED, "B*H*n too large");
  const size_t nin = (size_t)rows * a->d * (a->dtype == LLA_DTYPE_F32 ? 4 : 2);
  const size_t nf = (size_t)rows * a->d * 4, nrow = (size_t)rows * 4;
  struct Buf { const void* p; size_t bytes; const char* name; };
  const Buf ins[6] = {{a->q, nin, "q"},     {a->k, nin, "k"},       {a->v, nin, "v"},
                      {a->out, nf, "out"},  {a->dout, nf, "dout"},  {a->rho_c, nf, "rho_c"}};
  for (const Buf& in : ins)
    if (!aligned16(in.p)) return fail(LLA_ERR_INVALID_ARG, "%s pointer %p not 16-byte aligned", in.name, in.p);
  const Buf outs[5] = {{a->dq, nf, "dq"}, {a->dk, nf, "dk"}, {a->dv, nf, "dv"},
                       {a->adj_iters, nrow, "adj_iters"}, {a->adj_resid, nrow, "adj_resid"}};
  for (int i = 0; i < 5; ++i) {
    if (!outs[i].p) continue;
    if (!aligned16(outs[i].p))
      return fail(LLA_ERR_INVALID_ARG, "%s pointer %p not 16-byte aligned", outs[i].name, outs[i].p);
    for (const Buf& in : ins)
      if (overlap(outs[i].p, outs[i].bytes, in.p, in.bytes))
        return fail(LLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, in.name);
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
        return fail(LLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  if (a->workspace && !aligned16(a->workspace))
    return fail(LLA_ERR_INVALID_ARG, "workspace pointer not 16-byte aligned");
  if (a->flags & ~(LLA_FLAG_SPLIT_U | LLA_FLAG_PRECOND | LLA_FLAG_NO_PRECOND))
    return fail(LLA_ERR_INVALID_ARG, "unknown flags 0x%x", a->flags);
  if ((a->flags & LLA_FLAG_PRECOND) && (a->flags & LLA_FLAG_NO_PRECOND))
    return fail(LLA_ERR_INVALID_ARG, "LLA_FLAG_PRECOND and LLA_FLAG_NO_PRECOND together");
  lla::BwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.out = a->out; p.dout = a->dout; p.rho_c = a->rho_c;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.adj_iters = a->adj_iters; p.adj_resid = a->adj_resid;
  p.BH = (int)bh; p.n = a->n; p.d = a->d; p.dtype = a->dtype;
  p.lambda = a->lambda; p.cg_max_iters = a->cg_max_iters; p.cg_rel_tol = a->cg_rel_tol;
  p.flags = a->flags;
  p.ev_main_begin = a->ev_main_begin;
  p.ev_main_end = a->ev_main_end;
  if (kernel == LLA_KERNEL_VALU) {
    const hipError_t e = lla::launch_valu_bwd(p, stream);
    if (e != hipSuccess) return fail(LLA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return LLA_OK;
  }
  const size_t need = lla::bwd_workspace_bytes(p.BH, p.n, p.d);
  void* ws = a->workspace;
  bool owned = false;
  if (ws) {
    if (a->workspace_bytes < need)
      return fail(LLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", a->workspace_bytes, need);
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return fail(LLA_ERR_HIP, "workspace allocation of %zu bytes: %s", need,
                                     hipGetErrorString(e));
    owned = true;
  }
  p.workspace = ws;
  p.workspace_bytes = owned ? need : a->workspace_bytes;
  const hipError_t e = lla::launch_bwd(p, stream);
  if (owned) {
    const hipError_t f = hipFreeAsync(ws, stream);
    if (e == hipSuccess && f != hipSuccess)
      return fail(LLA_ERR_HIP, "workspace free: %s", hipGetErrorString(f));
  }
  if (e != hipSuccess) return fail(LLA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return LLA_OK;
}

size_t lla_backward_workspace_bytes(int B, int H, int n, int d, int dtype) {
  if (B < 1 || H < 1 || n < 1 || n > lla::kMfmaMaxN || !lla::mfma_supported(dtype, d)) return 0;  // (vector path: none)
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 0x7fffffffULL || bh * (unsigned long long)n > (1ULL << 40)) return 0;
  return lla::bwd_workspace_bytes((int)bh, n, d);
}

int lla_forward_f32(const float* q, const float* k, const float* v, float* out, int B, int H, int n,
                    int d, float lambda, int cg_max_iters, float cg_rel_tol, hipStream_t stream) {
  lla_fwd_args a{};
  a.dtype = LLA_DTYPE_F32;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.B = B; a.H = H; a.n = n; a.d = d;
  a.lambda = lambda; a.cg_max_iters = cg_max_iters; a.cg_rel_tol = cg_rel_tol;
  return lla_forward_ex(&a, stream);
}

int lla_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, int B, int H,
                     int n, int d, float lambda, int cg_max_iters, float cg_rel_tol,
                     hipStream_t stream) {
  lla_fwd_args a{};
  a.dtype = LLA_DTYPE_BF16;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.B = B; a.H = H; a.n = n; a.d = d;
  a.lambda = lambda; a.cg_max_iters = cg_max_iters; a.cg_rel_tol = cg_rel_tol;
  return lla_forward_ex(&a, stream);
}

}  // extern "C"
