// Internal declarations shared by the host API and the kernel translation
// units of liblla.so. Not part of the public ABI (see include/lla.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lla.h"

namespace lla {

// Everything a forward launch needs, already validated by the host API.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  float* omega;      // optional [BH][n]
  float* rho;        // optional [BH][n][d]
  float* rowmax;     // optional [BH][n]
  int32_t* cg_iters; // optional [BH][n]
  float* cg_resid;   // optional [BH][n]
  const float* rho_in;  // supplied rho_i [BH][n][d] (skips the CG solve), or NULL
  float* rho_c;      // optional [BH][n][d]: the centred system's solution
  int BH;            // B * H
  int n;
  int d;
  int dtype;         // LLA_DTYPE_*
  float lambda;
  int cg_max_iters;
  float cg_rel_tol;
  int flags;
  void* workspace;   // device scratch (kernel specific), may be NULL
  size_t workspace_bytes;
  hipEvent_t ev_main_begin;  // optional, recorded around the main kernel
  hipEvent_t ev_main_end;
};

// Everything a decode launch needs, already validated by the host API.
struct DecodeParams {
  const void* q;     // [BH][d]
  const void* k;     // [BH][n][d]
  const void* v;     // [BH][n][d]
  float* out;        // [BH][d]
  float* omega;      // optional [BH]
  float* rho;        // optional [BH][d]
  float* rowmax;     // optional [BH]
  int32_t* cg_iters; // optional [BH]
  float* cg_resid;   // optional [BH]
  int BH, n, d, dtype;
  float lambda;
  int cg_max_iters;
  float cg_rel_tol;
  void* workspace;
  size_t workspace_bytes;
  hipEvent_t ev_main_begin;  // optional, recorded around the main kernel (bf16: the one
                             // pass over the cache; fp32: the Gram kernel)
  hipEvent_t ev_main_end;
};

// decode-shaped forward (one query per head against n keys): d in {64,128},
// fp32 or bf16 inputs
bool decode_supported(int d);
size_t decode_workspace_bytes(int BH, int n, int d, int dtype);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// Static per-device scratch of lla_decode_noalloc: its size, and its device
// address on the current device (looked up once per device, then cached).
constexpr size_t kDecodeScratchBytes = LLA_DECODE_NOALLOC_SCRATCH_BYTES;
hipError_t decode_scratch(void** ptr);

// fp32 vector-ALU kernel (any d in {16,32,64,128}, fp32 or bf16 inputs).
hipError_t launch_valu(const FwdParams& p, hipStream_t stream);

// fp16 matrix-core kernel (bf16 inputs, d in {64,128}, n <= kMfmaMaxN: the
// byte offset of a head's last key tile, formed in 32-bit int arithmetic,
// stays below 2^31).
constexpr int kMfmaMaxN = 1 << 21;
size_t mfma_workspace_bytes(int BH, int n, int d);
bool mfma_supported(int dtype, int d);
hipError_t launch_mfma(const FwdParams& p, hipStream_t stream);
// Pieces of the matrix-core forward that its gradient reuses on the same
// workspace: the prepasses and the moment kernel (per-query kbar, omega, row
// max; the residual slab set to mu), and the CG kernel alone, which solves
// Sigma_c x = r for whatever right-hand side r the residual slab holds.
hipError_t mfma_moments(const FwdParams& p, bool two_term, hipStream_t stream);
// The preconditioners of the CG kernel (no-op when the call's flags and
// tolerance leave CG unpreconditioned), and the CG kernel, which uses them
// under the same rule (LLA_FLAG_PRECOND, LLA_FLAG_NO_PRECOND, else
// cg_rel_tol > 0).
hipError_t mfma_precond_build(const FwdParams& p, hipStream_t stream);
hipError_t mfma_cg(const FwdParams& p, hipStream_t stream);

// The naive forward (fp32; pairwise differences and moment matrices held in
// the workspace, exact Cholesky solves): its workspace and launch.
size_t naive_workspace_bytes(int BH, int n, int d);
hipError_t launch_naive(const FwdParams& p, hipStream_t stream);

// Everything a backward launch needs, already validated by the host API.
struct BwdParams {
  const void* q;      // bf16 [BH][n][d]
  const void* k;
  const void* v;
  const float* out;   // the forward output b [BH][n][d]
  const float* dout;  // dL/db [BH][n][d]
  const float* rho_c; // the forward's centred solution [BH][n][d]
  float* dq;          // [BH][n][d]
  float* dk;
  float* dv;
  int32_t* adj_iters; // optional [BH][n]: CG steps of the adjoint solve
  float* adj_resid;   // optional [BH][n]
  int BH, n, d, dtype;
  float lambda;
  int cg_max_iters;
  float cg_rel_tol;
  int flags;         // LLA_FLAG_SPLIT_U: U of the adjoint products as two fp16 terms
  void* workspace;
  size_t workspace_bytes;
  hipEvent_t ev_main_begin;  // optional, recorded around the adjoint CG kernel
  hipEvent_t ev_main_end;
};

// gradient of the matrix-core forward (bf16 inputs, d in {64,128})
size_t bwd_workspace_bytes(int BH, int n, int d);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);
// gradient of the vector-ALU forward (fp32 or bf16 inputs, d in {16,32,64,128});
// no workspace; dk and dv are zero-filled and accumulated with atomics
hipError_t launch_valu_bwd(const BwdParams& p, hipStream_t stream);

}  // namespace lla
