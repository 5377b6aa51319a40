// ssm_scan.hip -- C ABI of the gfx950 selective state-space scan.
//
// Entry points are declared (with their contracts) in include/ssm_scan.h.
// This file validates arguments before any HIP call, plans the launch
// (states per lane, wavefronts per workgroup, number of sequence chunks) and
// enqueues the kernels of scan_kernels.hpp / decode_kernel.hpp on the
// caller's stream.  It allocates nothing and keeps no state.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "decode_kernel.hpp"
#include "scan_kernels.hpp"

namespace ssm {
namespace {

constexpr int64_t kMaxGrid = 65535;  // limit for grid.y (batch) and grid.z (chunks)
constexpr int64_t kChunkQuantum = 32; // chunk lengths are multiples of the largest token block
constexpr int64_t kMinChunk = 256;    // never cut the sequence finer than this
constexpr int kTargetWaves = 2048;    // aim for ~2 wavefronts per SIMD (256 CUs x 4 SIMDs)

struct Plan {
  int npl;       // states per lane
  int G;         // wavefronts per workgroup (state groups)
  int K;         // sequence chunks
  int64_t chunk_len;
  size_t ws_bytes;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int next_pow2(int64_t x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Optional override for tuning experiments: SSM_SCAN_VARIANT="npl,G[,K]".
bool env_variant(int* npl, int* G, int* K) {
  const char* s = getenv("SSM_SCAN_VARIANT");
  if (!s || !*s) return false;
  int a = 0, b = 0, k = 0;
  const int n = sscanf(s, "%d,%d,%d", &a, &b, &k);
  if (n < 2) return false;
  *npl = a;
  *G = b;
  *K = (n >= 3) ? k : 0;
  return true;
}

bool variant_exists(int npl, int G) {
  if (npl == 4 && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16)) return true;
  if ((npl == 2 && G == 8) || (npl == 1 && G == 16) || (npl == 8 && G == 2) || (npl == 16 && G == 1)) return true;
  return false;
}

void plan_scan(int64_t batch, int64_t L, int64_t dim, int64_t N, Plan* pl) {
  int npl, G, Kreq = 0;
  if (N == 16) {
    npl = 2;
    G = 8;
  } else {
    npl = 4;
    G = next_pow2(ceil_div(N, 4));
  }
  int enpl, eG, eK;
  if (env_variant(&enpl, &eG, &eK) && variant_exists(enpl, eG) && static_cast<int64_t>(enpl) * eG >= N) {
    npl = enpl;
    G = eG;
    Kreq = eK;
  }
  const int64_t tiles = batch * ceil_div(dim, 64);
  int64_t K = Kreq > 0 ? Kreq : ceil_div(kTargetWaves, tiles * G);
  const int64_t kmax = ceil_div(L, kMinChunk);
  if (Kreq <= 0 && K > kmax) K = kmax;
  if (K < 1) K = 1;
  int64_t chunk = ceil_div(ceil_div(L, K), kChunkQuantum) * kChunkQuantum;
  K = ceil_div(L, chunk);
  pl->npl = npl;
  pl->G = G;
  pl->K = static_cast<int>(K > kMaxGrid + 1 ? kMaxGrid + 1 : K);
  pl->chunk_len = chunk;
  pl->ws_bytes = 0;
  if (K > 1) {
    const size_t one = align256(static_cast<size_t>(batch) * K * dim * N * sizeof(float));
    pl->ws_bytes = 3 * one;
  }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ssm_status_t check_scan_args(const void* u, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* bias, void* y, float* fs,
                             int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt) {
  if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0) return SSM_ERR_INVALID_ARG;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return SSM_ERR_INVALID_ARG;
  const size_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(y, es) || (z && !aligned(z, es))) return SSM_ERR_INVALID_ARG;
  if (!aligned(B, 4) || !aligned(C, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) || (bias && !aligned(bias, 4)) ||
      (fs && !aligned(fs, 4)))
    return SSM_ERR_INVALID_ARG;
  if (dstate > 64) return SSM_ERR_UNSUPPORTED;
  if (dt == SSM_DTYPE_BF16 && (dstate & 1)) return SSM_ERR_UNSUPPORTED;
  if (batch > kMaxGrid) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

template <class IO, int VW, bool FULL>
hipError_t launch_scan(int npl, int G, bool exact, const ScanParams& p, dim3 grid, hipStream_t s) {
#define SSM_SCAN_CASE(NPL_, G_, EX_)                                                                \
  if (npl == NPL_ && G == G_ && exact == EX_) {                                                   \
    hipLaunchKernelGGL((scan_kernel<IO, NPL_, G_, VW, FULL, (EX_ ? NPL_ * G_ : 0)>), grid,         \
                       dim3(64 * G_), 0, s, p);                                                   \
    return hipGetLastError();                                                                     \
  }
  if constexpr (VW == 4) {
    SSM_SCAN_CASE(4, 1, true)
    SSM_SCAN_CASE(4, 2, true)
    SSM_SCAN_CASE(4, 4, true)
    SSM_SCAN_CASE(4, 8, true)
    SSM_SCAN_CASE(4, 1, false)
    SSM_SCAN_CASE(4, 2, false)
    SSM_SCAN_CASE(4, 4, false)
    SSM_SCAN_CASE(4, 8, false)
    SSM_SCAN_CASE(2, 8, true)
    SSM_SCAN_CASE(8, 2, true)
    SSM_SCAN_CASE(16, 1, true)
  } else {
    SSM_SCAN_CASE(4, 1, true)
    SSM_SCAN_CASE(4, 2, true)
    SSM_SCAN_CASE(4, 4, true)
    SSM_SCAN_CASE(4, 8, true)
    SSM_SCAN_CASE(4, 16, true)
    SSM_SCAN_CASE(4, 1, false)
    SSM_SCAN_CASE(4, 2, false)
    SSM_SCAN_CASE(4, 4, false)
    SSM_SCAN_CASE(4, 8, false)
    SSM_SCAN_CASE(4, 16, false)
    SSM_SCAN_CASE(1, 16, true)
  }
#undef SSM_SCAN_CASE
  return hipErrorInvalidValue;
}

template <class IO>
hipError_t run_scan(const Plan& pl, bool vec4, const ScanParams& p, hipStream_t s) {
  const bool exact = static_cast<int64_t>(pl.npl) * pl.G == p.N;
  const dim3 grid_full(static_cast<unsigned>(ceil_div(p.dim, 64)), static_cast<unsigned>(p.batch),
                       static_cast<unsigned>(pl.K));
  hipError_t e = hipSuccess;
  if (pl.K > 1) {
    const dim3 grid_agg(grid_full.x, grid_full.y, static_cast<unsigned>(pl.K - 1));
    e = vec4 ? launch_scan<IO, 4, false>(pl.npl, pl.G, exact, p, grid_agg, s)
             : launch_scan<IO, 1, false>(pl.npl, pl.G, exact, p, grid_agg, s);
    if (e != hipSuccess) return e;
    const int64_t DN = p.dim * p.N;
    const int64_t threads = p.batch * DN;
    hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>(ceil_div(threads, 256))), dim3(256), 0, s,
                       static_cast<const float*>(p.aggP), static_cast<const float*>(p.aggS), p.carry, p.batch,
                       pl.K, DN);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return vec4 ? launch_scan<IO, 4, true>(pl.npl, pl.G, exact, p, grid_full, s)
              : launch_scan<IO, 1, true>(pl.npl, pl.G, exact, p, grid_full, s);
}

template <class IO>
hipError_t run_decode(const DecodeParams& p, hipStream_t s) {
  const int nq = next_pow2(ceil_div(p.N, 4));
  const bool vec4 = (p.N % 4) == 0 && aligned(p.state, 16) && aligned(p.A, 16);
  const int64_t threads = p.batch * p.dim * nq;
  const dim3 grid(static_cast<unsigned>(ceil_div(threads, 256)));
#define SSM_DEC_CASE(NQ_)                                                                         \
  if (nq == NQ_) {                                                                                \
    if (vec4)                                                                                     \
      hipLaunchKernelGGL((state_update_kernel<IO, NQ_, true>), grid, dim3(256), 0, s, p);         \
    else                                                                                          \
      hipLaunchKernelGGL((state_update_kernel<IO, NQ_, false>), grid, dim3(256), 0, s, p);        \
    return hipGetLastError();                                                                     \
  }
  SSM_DEC_CASE(1)
  SSM_DEC_CASE(2)
  SSM_DEC_CASE(4)
  SSM_DEC_CASE(8)
  SSM_DEC_CASE(16)
#undef SSM_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" size_t ssm_scan_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt) {
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > 64 || batch > kMaxGrid) return 0;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return 0;
  if (dt == SSM_DTYPE_BF16 && (dstate & 1)) return 0;
  Plan pl;
  plan_scan(batch, L, dim, dstate, &pl);
  return pl.ws_bytes;
}

extern "C" ssm_status_t ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                     const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                     void* y, float* final_state, int64_t batch, int64_t L, int64_t dim,
                                     int64_t dstate, ssm_dtype_t dt, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  const ssm_status_t st =
      check_scan_args(u, delta, A, B, C, D, z, delta_bias, y, final_state, batch, L, dim, dstate, dt);
  if (st != SSM_OK) return st;
  Plan pl;
  plan_scan(batch, L, dim, dstate, &pl);
  if (pl.K > kMaxGrid) return SSM_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !aligned(workspace, 256)))
    return SSM_ERR_INVALID_ARG;

  ScanParams p;
  p.u = u;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.y = y;
  p.final_state = final_state;
  p.batch = batch;
  p.L = L;
  p.dim = dim;
  p.N = dstate;
  p.chunk_len = pl.chunk_len;
  p.K = pl.K;
  p.softplus = softplus_flag ? 1 : 0;
  p.aggP = p.aggS = p.carry = nullptr;
  if (pl.K > 1) {
    const size_t one = pl.ws_bytes / 3;
    char* ws = static_cast<char*>(workspace);
    p.aggP = reinterpret_cast<float*>(ws);
    p.aggS = reinterpret_cast<float*>(ws + one);
    p.carry = reinterpret_cast<float*>(ws + 2 * one);
  }
  // Vector (4-wide) prologue/epilogue needs dim % 4 == 0 and aligned token rows.
  const size_t vbytes = dt == SSM_DTYPE_F32 ? 16 : 8;
  bool vec4 = (dim % 4) == 0 && aligned(u, vbytes) && aligned(delta, vbytes) && aligned(y, vbytes) &&
              (!z || aligned(z, vbytes));
  // Variants with 16 wavefronts only exist with the 1-wide prologue.
  if (pl.G == 16) vec4 = false;
  // The 1-wide family is the (npl = 4) one plus (1, 16); fall back to it when needed.
  if (!vec4 && !(pl.npl == 4 || (pl.npl == 1 && pl.G == 16))) {
    pl.npl = 4;
    pl.G = next_pow2(ceil_div(dstate, 4));
  }
  const hipError_t e = dt == SSM_DTYPE_F32 ? run_scan<F32>(pl, vec4, p, stream) : run_scan<BF16>(pl, vec4, p, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" ssm_status_t ssm_state_update(float* state, const void* u, const void* delta, const float* A,
                                         const void* B, const void* C, const float* D, const void* z,
                                         const float* delta_bias, int softplus_flag, void* y, int64_t batch,
                                         int64_t dim, int64_t dstate, ssm_dtype_t dt, hipStream_t stream) {
  if (!state || !u || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  if (batch <= 0 || dim <= 0 || dstate <= 0) return SSM_ERR_INVALID_ARG;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return SSM_ERR_INVALID_ARG;
  const size_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(y, es) || !aligned(B, es) || !aligned(C, es) ||
      (z && !aligned(z, es)) || !aligned(state, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)))
    return SSM_ERR_INVALID_ARG;
  if (dstate > 64) return SSM_ERR_UNSUPPORTED;
  const int64_t threads = batch * dim * next_pow2(ceil_div(dstate, 4));
  if (ceil_div(threads, 256) > 0x7fffffff) return SSM_ERR_UNSUPPORTED;
  DecodeParams p;
  p.state = state;
  p.u = u;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.y = y;
  p.batch = batch;
  p.dim = dim;
  p.N = dstate;
  p.softplus = softplus_flag ? 1 : 0;
  const hipError_t e = dt == SSM_DTYPE_F32 ? run_decode<F32>(p, stream) : run_decode<BF16>(p, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" const char* ssm_status_string(ssm_status_t s) {
  switch (s) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
    case SSM_ERR_HIP: return "SSM_ERR_HIP";
  }
  return "SSM_ERR_UNKNOWN";
}
