// ssm_scan.hip -- C ABI of the gfx950 selective state-space scan.
//
// Entry points are declared (with their contracts) in include/ssm_scan.h.
// This file validates arguments before any HIP call, plans the launch
// (states per lane, wavefronts per workgroup, which tiles are cut into
// sequence chunks) and enqueues the kernels of scan_kernels.hpp and
// decode_kernel.hpp on the caller's stream.  It allocates nothing and keeps
// no state.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "decode_kernel.hpp"
#include "scan_kernels.hpp"

namespace ssm {
namespace {

constexpr int64_t kMaxBatch = 65535;
constexpr int64_t kChunkQuantum = kTrip;  // chunk lengths are multiples of the main loop trip
constexpr int64_t kMinChunk = 256;        // never cut the sequence finer than this
constexpr int64_t kNumCU = 256;           // MI355X compute units: the work is balanced over these
constexpr int64_t kMaxChunks = 4096;      // chunks per split tile

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int next_pow2(int64_t x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Plan {
  int vw;        // channels per prologue/epilogue thread (vector width of the token-row accesses)
  int npl;       // states per lane
  int G;         // wavefronts per workgroup (state groups); npl * G >= dstate
  int ntd;       // 64-channel tiles per batch row
  int n_long;    // tiles scanned whole
  int n_split;   // tiles cut into Ks chunks
  int Ks;        // chunks per split tile
  int64_t chunk_len;
  int64_t Lp;    // sequence length rounded up to whole token blocks (packed B/C rows)
  bool touch;    // L2 touch of upcoming B/C records (scan_kernel's TOUCH)
};

// Workspace layout: [packed B/C][chunk fades P][chunk states S][carried-in states].
struct Layout {
  size_t bc, agg, total;
};

Layout layout_for(const Plan& pl, int64_t batch) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.G;
  Layout l;
  l.bc = align256((static_cast<size_t>(batch) * pl.Lp + kTB) * 2 * npad * sizeof(float));
  l.agg = pl.n_split > 0 ? align256(static_cast<size_t>(pl.n_split) * pl.Ks * 64 * npad * sizeof(float)) : 0;
  l.total = l.bc + 3 * l.agg;
  return l;
}

// Optional override for tuning experiments: SSM_SCAN_VARIANT="npl,G[,K]".
// K > 0 cuts every tile into K chunks; K = 0 (or absent) keeps the planner's split.
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

// Kernel variants (states per lane, wavefronts).  Each exists with its
// preferred prologue width (channels per thread: 4 up to 4 wavefronts, 2 for
// 8, 1 for 16) and with width 1.
bool variant_exists(int npl, int G) {
  if (npl == 4 && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16)) return true;
  return (npl == 2 && G == 8) || (npl == 1 && G == 16) || (npl == 8 && G == 2) || (npl == 16 && G == 1);
}
int preferred_vw(int G) { return G <= 4 ? 4 : (G == 8 ? 2 : 1); }

// The generic variant for a state size: 4 states per lane, a power of two of wavefronts.
void generic_variant(int64_t N, int* npl, int* G) {
  *npl = 4;
  *G = next_pow2(ceil_div(N, 4));
}

// The kernels address a chunk's token rows with 32-bit byte offsets: a chunk
// (plus one trip of padding) must stay below 2^31 bytes per tensor, so very
// long rows force every tile to be cut.
int64_t max_chunk_len(int64_t dim, int64_t es) {
  return (0x7fffffffLL / (dim * es) - kTrip) / kTrip * kTrip;
}

// Work plan.  A tile (64 channels of one batch row) scanned whole costs one
// pass over L tokens; cutting it into chunks adds an aggregate pass over all
// but its last chunk (about four fifths of the cost per token), so tiles are
// only cut when there are too few of them to keep the GPU busy: with at least
// 3/4 as many tiles as CUs every tile runs whole; otherwise every tile is cut
// so that each CU gets about two chunks (two workgroups of the 16-state
// variant fit on a CU).
// vw_ok: the widest token-row access the pointers and dim allow (4, 2 or 1);
// it decides the prologue width, not the split.
void plan_scan(int64_t batch, int64_t L, int64_t dim, int64_t N, int64_t es, int vw_ok, Plan* pl) {
  int npl, G, Kreq = 0;
  if (N == 16) {
    // 2 states per lane over 8 wavefronts: 80 KB of LDS, two workgroups per CU.
    npl = 2;
    G = 8;
  } else {
    generic_variant(N, &npl, &G);
  }
  int enpl, eG, eK;
  if (env_variant(&enpl, &eG, &eK) && variant_exists(enpl, eG) && static_cast<int64_t>(enpl) * eG >= N) {
    npl = enpl;
    G = eG;
    Kreq = eK;
  }
  const int vw = preferred_vw(G) <= vw_ok ? preferred_vw(G) : 1;
  const int64_t ntd = ceil_div(dim, 64);
  const int64_t T = batch * ntd;
  const int64_t kmax = ceil_div(L, kMinChunk) < kMaxChunks ? ceil_div(L, kMinChunk) : kMaxChunks;
  int64_t n_long, K;
  if (Kreq > 0) {
    K = Kreq;
    n_long = 0;
  } else if (4 * T >= 3 * kNumCU) {
    n_long = T;
    K = 1;
  } else {
    n_long = 0;
    K = ceil_div(2 * kNumCU, T);
    if (K > kmax) K = kmax;
  }
  if (K < 1) K = 1;
  const int64_t kmin = ceil_div(L, max_chunk_len(dim, es));
  if (kmin > 1) {
    n_long = 0;
    if (K < kmin) K = kmin;
  }
  int64_t chunk = ceil_div(ceil_div(L, K), kChunkQuantum) * kChunkQuantum;
  K = ceil_div(L, chunk);
  if (K == 1) n_long = T;
  pl->vw = vw;
  pl->npl = npl;
  pl->G = G;
  pl->ntd = static_cast<int>(ntd);
  pl->n_long = static_cast<int>(n_long);
  pl->n_split = static_cast<int>(T - n_long);
  pl->Ks = static_cast<int>(K);
  pl->chunk_len = chunk;
  pl->Lp = ceil_div(L, kTrip) * kTrip;
  // With fewer tiles than CUs a CU holds one workgroup and the scalar loads'
  // latency is exposed (or the records stream from HBM): touch them into L2.
  pl->touch = T < kNumCU;
  const char* te = getenv("SSM_SCAN_TOUCH");  // tuning override: "0" or "1"
  if (te && (te[0] == '0' || te[0] == '1')) pl->touch = te[0] == '1';
}

ssm_status_t check_scan_args(const void* u, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* bias, void* y, float* fs,
                             int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt) {
  if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0) return SSM_ERR_INVALID_ARG;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return SSM_ERR_INVALID_ARG;
  const size_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(y, es) || (z && !aligned(z, es)) || !aligned(B, es) ||
      !aligned(C, es))
    return SSM_ERR_INVALID_ARG;
  if (!aligned(A, 4) || (D && !aligned(D, 4)) || (bias && !aligned(bias, 4)) || (fs && !aligned(fs, 4)))
    return SSM_ERR_INVALID_ARG;
  if (dstate > 64) return SSM_ERR_UNSUPPORTED;
  if (batch > kMaxBatch) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

template <class IO, bool FULL>
hipError_t launch_scan(int npl, int G, int vw, bool touch, const ScanParams& p, dim3 grid, hipStream_t s) {
#define SSM_SCAN_LAUNCH(NPL_, G_, VW_)                                                                     \
  if (touch)                                                                                             \
    hipLaunchKernelGGL((scan_kernel<IO, NPL_, G_, VW_, FULL, true>), grid, dim3(64 * G_), 0, s, p);       \
  else                                                                                                   \
    hipLaunchKernelGGL((scan_kernel<IO, NPL_, G_, VW_, FULL, false>), grid, dim3(64 * G_), 0, s, p);
#define SSM_SCAN_CASE(NPL_, G_)                                                                            \
  if (npl == NPL_ && G == G_) {                                                                          \
    constexpr int VWP = (G_ <= 4) ? 4 : ((G_ == 8) ? 2 : 1);                                             \
    if (vw == VWP) {                                                                                     \
      SSM_SCAN_LAUNCH(NPL_, G_, VWP)                                                                     \
    } else {                                                                                             \
      SSM_SCAN_LAUNCH(NPL_, G_, 1)                                                                       \
    }                                                                                                    \
    return hipGetLastError();                                                                            \
  }
  SSM_SCAN_CASE(4, 1)
  SSM_SCAN_CASE(4, 2)
  SSM_SCAN_CASE(4, 4)
  SSM_SCAN_CASE(4, 8)
  SSM_SCAN_CASE(4, 16)
  SSM_SCAN_CASE(2, 8)
  SSM_SCAN_CASE(1, 16)
  SSM_SCAN_CASE(8, 2)
  SSM_SCAN_CASE(16, 1)
#undef SSM_SCAN_CASE
#undef SSM_SCAN_LAUNCH
  return hipErrorInvalidValue;
}

template <class IO>
hipError_t run_scan(const Plan& pl, const void* B, const void* C, float* bc, ScanParams p, hipStream_t s) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.G;
  const dim3 pgrid(static_cast<unsigned>(p.batch * (pl.Lp / kPackT)));
#define SSM_PACK_CASE(NPL_)                                                                                  \
  if (pl.npl == NPL_)                                                                                       \
    hipLaunchKernelGGL((pack_bc_kernel<IO, NPL_>), pgrid, dim3(256), 0, s, B, C, bc, p.batch, p.L, pl.Lp, p.N, \
                       pl.G);
  SSM_PACK_CASE(1)
  SSM_PACK_CASE(2)
  SSM_PACK_CASE(4)
  SSM_PACK_CASE(8)
  SSM_PACK_CASE(16)
#undef SSM_PACK_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.n_split > 0 && pl.Ks > 1) {
    const dim3 grid_agg(static_cast<unsigned>(static_cast<int64_t>(pl.n_split) * (pl.Ks - 1)));
    e = launch_scan<IO, false>(pl.npl, pl.G, pl.vw, pl.touch, p, grid_agg, s);
    if (e != hipSuccess) return e;
    const int64_t cols = static_cast<int64_t>(pl.n_split) * 64 * npad;
    hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>(ceil_div(cols, kCarryCols))), dim3(256), 0, s,
                       static_cast<const float*>(p.aggP), static_cast<const float*>(p.aggS), p.carry,
                       static_cast<int64_t>(pl.n_split), pl.Ks, npad);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid_full(static_cast<unsigned>(pl.n_long + static_cast<int64_t>(pl.n_split) * pl.Ks));
  return launch_scan<IO, true>(pl.npl, pl.G, pl.vw, pl.touch, p, grid_full, s);
}

template <class IO>
hipError_t run_decode(const DecodeParams& p, hipStream_t s) {
  const int nq = next_pow2(ceil_div(p.N, 4));
  const size_t es = __is_same(IO, F32) ? 4 : 2;
  const bool vec4 = (p.N % 4) == 0 && aligned(p.state, 16) && aligned(p.A, 16);
  if (vec4 && aligned(p.B, 4 * es) && aligned(p.C, 4 * es)) {
    // R batch rows per thread: A, bias and D are then read once per R rows.
    const int R = p.batch >= 4 ? 4 : (p.batch >= 2 ? 2 : 1);
    const int64_t threads = ceil_div(p.batch, R) * p.dim * nq;
    const dim3 grid(static_cast<unsigned>(ceil_div(threads, 256)));
#define SSM_DECV_CASE(NQ_)                                                                         \
  if (nq == NQ_) {                                                                                 \
    if (R == 4)                                                                                    \
      hipLaunchKernelGGL((state_update_vec_kernel<IO, NQ_, 4>), grid, dim3(256), 0, s, p);         \
    else if (R == 2)                                                                               \
      hipLaunchKernelGGL((state_update_vec_kernel<IO, NQ_, 2>), grid, dim3(256), 0, s, p);         \
    else                                                                                           \
      hipLaunchKernelGGL((state_update_vec_kernel<IO, NQ_, 1>), grid, dim3(256), 0, s, p);         \
    return hipGetLastError();                                                                      \
  }
    SSM_DECV_CASE(1)
    SSM_DECV_CASE(2)
    SSM_DECV_CASE(4)
    SSM_DECV_CASE(8)
    SSM_DECV_CASE(16)
#undef SSM_DECV_CASE
    return hipErrorInvalidValue;
  }
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
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > 64 || batch > kMaxBatch) return 0;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return 0;
  // The packed layout depends only on the variant, which the pointers do not
  // change; size it for the widest and the narrowest prologue anyway.
  Plan p4, p1;
  const int64_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  if (max_chunk_len(dim, es) < kChunkQuantum) return 0;
  plan_scan(batch, L, dim, dstate, es, 4, &p4);
  plan_scan(batch, L, dim, dstate, es, 1, &p1);
  const size_t a = layout_for(p4, batch).total, b = layout_for(p1, batch).total;
  return a > b ? a : b;
}

extern "C" ssm_status_t ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                     const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                     void* y, float* final_state, int64_t batch, int64_t L, int64_t dim,
                                     int64_t dstate, ssm_dtype_t dt, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  const ssm_status_t st =
      check_scan_args(u, delta, A, B, C, D, z, delta_bias, y, final_state, batch, L, dim, dstate, dt);
  if (st != SSM_OK) return st;
  // A prologue width vw needs dim % vw == 0 and token rows aligned to vw elements.
  const size_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  int vw_ok = 1;
  for (int v = 4; v >= 2; v /= 2) {
    const size_t vb = es * v;
    if ((dim % v) == 0 && aligned(u, vb) && aligned(delta, vb) && aligned(y, vb) && (!z || aligned(z, vb))) {
      vw_ok = v;
      break;
    }
  }
  if (max_chunk_len(dim, static_cast<int64_t>(es)) < kChunkQuantum) return SSM_ERR_UNSUPPORTED;
  Plan pl;
  plan_scan(batch, L, dim, dstate, static_cast<int64_t>(es), vw_ok, &pl);
  if (static_cast<int64_t>(pl.n_long) + static_cast<int64_t>(pl.n_split) * pl.Ks > 0x7fffffffLL ||
      batch * (pl.Lp / kPackT) > 0x7fffffffLL)
    return SSM_ERR_UNSUPPORTED;
  const Layout lay = layout_for(pl, batch);
  if (!workspace || workspace_bytes < lay.total || !aligned(workspace, 256)) return SSM_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  ScanParams p;
  p.u = u;
  p.delta = delta;
  p.A = A;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.bc = reinterpret_cast<const float*>(ws);
  p.y = y;
  p.final_state = final_state;
  p.aggP = p.aggS = p.carry = nullptr;
  if (pl.n_split > 0) {
    p.aggP = reinterpret_cast<float*>(ws + lay.bc);
    p.aggS = reinterpret_cast<float*>(ws + lay.bc + lay.agg);
    p.carry = reinterpret_cast<float*>(ws + lay.bc + 2 * lay.agg);
  }
  p.batch = batch;
  p.L = L;
  p.Lp = pl.Lp;
  p.dim = dim;
  p.N = dstate;
  p.chunk_len = pl.chunk_len;
  p.ntd = pl.ntd;
  p.n_long = pl.n_long;
  p.Ks = pl.Ks;
  p.softplus = softplus_flag ? 1 : 0;
  float* bc = reinterpret_cast<float*>(ws);
  const hipError_t e = dt == SSM_DTYPE_F32 ? run_scan<F32>(pl, B, C, bc, p, stream)
                                           : run_scan<BF16>(pl, B, C, bc, p, stream);
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
