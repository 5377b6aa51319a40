// ssm_scan.hip -- C ABI of the gfx950 selective state-space scan.
//
// Entry points are declared (with their contracts) in include/ssm_scan.h.
// This file validates arguments before any HIP call, plans the launch
// (states per lane, wavefronts per workgroup, which tiles are cut into
// sequence chunks) and enqueues the kernels of scan_kernels.hpp and
// decode_kernel.hpp on the caller's stream.  It allocates nothing and keeps
// no state beyond each device's compute-unit count, looked up once.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "carry_kernel.hpp"
#include "decode_kernel.hpp"
#include "host_common.hpp"
#include "lane_kernels.hpp"
#include "order_kernel.hpp"
#include "scan_launch.hpp"

namespace ssm {
namespace {

constexpr int64_t kMaxBatch = 65535;
constexpr int64_t kChunkQuantum = kTrip;  // chunk lengths are multiples of the main loop trip
constexpr int64_t kMinChunk = 256;        // never cut the sequence finer than this
constexpr int64_t kMaxChunks = 4096;      // chunks per split tile
constexpr int64_t kMaxChained = 8;        // chunks per tile in a chained launch (the carry hops in series)

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
  bool chained;  // split tiles chain their carries inside the one scan launch
  int tb;        // tokens per block of the readout scan (16, or 32 with a CU per workgroup)
  bool packed;   // packed sequences: "chunk" c of a tile column is sequence c (no pairs, no carries)
  bool trap;     // trapezoidal rule: also C_t . B_t per token
  bool direct;   // fp32 storage, two-term rule: the scan reads B and C directly (no packed records)
};

// Workspace layout: [header words (status, ticket, ...) and ready flags]
// [packed B/C][chunk fades P][chunk states S][carried-in states][sequence
// order][C_t . B_t].  The chained plan needs no P, S and has a flag per
// chunk; only the packed plan has an order, only the trapezoidal rule C . B;
// fp32 storage with the two-term rule packs no B/C.
struct Layout {
  size_t words, bc, pairs, carry, order, cb, total;
  int n_words;
};

Layout layout_for(const Plan& pl, int64_t batch) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.G;
  const size_t per = static_cast<size_t>(pl.n_split) * pl.Ks * 64 * npad * sizeof(float);
  Layout l;
  l.n_words = kHeaderWords + (pl.chained ? pl.n_split * pl.Ks : 0);
  l.words = align256(static_cast<size_t>(l.n_words) * sizeof(unsigned));
  l.bc = pl.direct ? 0 : align256((static_cast<size_t>(batch) * pl.Lp + kTBMax) * 2 * npad * sizeof(float));
  l.pairs = (pl.n_split > 0 && !pl.chained && !pl.packed) ? align256(per) : 0;
  l.carry = (pl.n_split > 0 && !pl.packed) ? align256(per) : 0;
  l.order = pl.packed ? align256(static_cast<size_t>(pl.Ks) * sizeof(int)) : 0;
  l.cb = pl.trap ? align256(static_cast<size_t>(batch) * (pl.Lp + kTBMax) * sizeof(float)) : 0;
  l.total = l.words + l.bc + 2 * l.pairs + l.carry + l.order + l.cb;
  return l;
}

// Optional overrides for tuning experiments and tests:
//   SSM_SCAN_VARIANT="npl,G[,K]"  K > 0 cuts every tile into K chunks; K = 0
//                                 (or absent) keeps the planner's split;
//   SSM_SCAN_CHAINED=0|1          chunks chain their carries in the scan launch
//                                 (1) or go through the pair and carry passes (0);
//   SSM_SCAN_CHAIN_K=k            chunks per left-over tile in a chained plan;
//   SSM_SCAN_TB=16|32             tokens per block of the readout scan, where
//                                 the variant has both;
//   SSM_SCAN_ORDER=0              packed sequences launch in index order rather
//                                 than longest first.
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

// The generic variant for a state size: 4 states per lane, a power of two of wavefronts.
void generic_variant(int64_t N, int* npl, int* G) {
  *npl = 4;
  *G = next_pow2(ceil_div(N, 4));
}

// The kernels address a chunk's token rows with 32-bit byte offsets: a chunk
// (plus one trip of padding) must stay below 2^31 bytes per tensor, so very
// long rows force every tile to be cut.  row_bytes: the larger of a token row
// of u (dim * element size) and, where the scan reads B and C directly, of B
// (dstate * 4).
int64_t max_chunk_len(int64_t row_bytes) {
  return (0x7fffffffLL / row_bytes - kTrip) / kTrip * kTrip;
}
int64_t token_row_bytes(int64_t dim, int64_t N, int64_t es, bool direct) {
  return (direct && N * 4 > dim * es) ? N * 4 : dim * es;
}

int env_flag(const char* name) {  // -1 when unset
  const char* v = getenv(name);
  return (v && (v[0] == '0' || v[0] == '1')) ? v[0] - '0' : -1;
}

// Work plan.  A tile (64 channels of one batch row) scanned whole costs one
// pass over L tokens; cutting it into chunks costs either a pass computing
// each chunk's pair (about as costly per token as the scan itself) or waiting
// for the chunk before it, so tiles are cut only where the GPU would
// otherwise run unevenly:
//   - up to half as many tiles again as CUs (the 2.8B-shaped layer: 320
//     tiles): one workgroup per CU runs one tile whole, and the r tiles left
//     over are cut into CUs/r chunks (at most kMaxChained), one spliced into
//     each workgroup's tile at the point where the chunk before it is done
//     (scan_kernel's chained mode);
//   - otherwise, with at least 3/4 as many tiles as CUs, every tile runs whole;
//   - with fewer tiles, every tile is cut so that each CU gets about two
//     chunks, through the separate pair and carry passes.
// vw_ok: the widest token-row access the pointers and dim allow (4, 2 or 1);
// it decides the prologue width, not the split.  rule: the discretisation
// (fp32 storage with the two-term rule reads B and C without packing them).
void plan_scan(int64_t batch, int64_t L, int64_t dim, int64_t N, int64_t es, int vw_ok, int rule, Plan* pl) {
  const int64_t kNumCU = device_cu_count();
  const bool direct = es == 4 && rule == kRuleEuler;
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
  const int env_chained = env_flag("SSM_SCAN_CHAINED");
  const int vw = preferred_vw(G) <= vw_ok ? preferred_vw(G) : 1;
  const int64_t ntd = ceil_div(dim, 64);
  const int64_t T = batch * ntd;
  const int64_t kmax = ceil_div(L, kMinChunk) < kMaxChunks ? ceil_div(L, kMinChunk) : kMaxChunks;
  int64_t n_long, K;
  bool chained = false;
  if (Kreq > 0 && env_chained == 1) {
    // forced chained plan: cut as many tiles r into Kreq chunks as leave one
    // chunk per whole-tile workgroup (r * K <= T - r)
    K = Kreq;
    int64_t r = T / (K + 1);
    if (r < 1) r = 1;
    n_long = T - r;
    chained = r * K <= n_long;
    if (!chained) n_long = 0;
  } else if (Kreq > 0) {
    K = Kreq;
    n_long = 0;
  } else if (T > kNumCU && 2 * (T - kNumCU) <= kNumCU && env_chained != 0) {
    const int64_t r = T - kNumCU;
    n_long = kNumCU;
    K = kNumCU / r;  // r * K <= kNumCU: one chunk per workgroup at most
    if (K < 2) K = 2;
    if (K > kMaxChained) K = kMaxChained;
    const char* ke = getenv("SSM_SCAN_CHAIN_K");  // tuning override of the chunk count
    if (ke && atoi(ke) >= 2) K = atoi(ke);
    if (r * K > n_long) K = n_long / r;  // at most one chunk per workgroup
    if (K > kmax) K = kmax;
    chained = true;
  } else if (4 * T >= 3 * kNumCU) {
    n_long = T;
    K = 1;
  } else {
    n_long = 0;
    K = ceil_div(2 * kNumCU, T);
    if (K > kmax) K = kmax;
  }
  if (K < 1) K = 1;
  const int64_t kmin = ceil_div(L, max_chunk_len(token_row_bytes(dim, N, es, direct)));
  if (kmin > 1) {
    n_long = 0;
    chained = false;
    if (K < kmin) K = kmin;
  }
  int64_t chunk = ceil_div(ceil_div(L, K), kChunkQuantum) * kChunkQuantum;
  K = ceil_div(L, chunk);
  if (K == 1) {
    n_long = T;
    chained = false;
  }
  pl->vw = vw;
  pl->npl = npl;
  pl->G = G;
  pl->ntd = static_cast<int>(ntd);
  pl->n_long = static_cast<int>(n_long);
  pl->n_split = static_cast<int>(T - n_long);
  pl->Ks = static_cast<int>(K);
  pl->chunk_len = chunk;
  pl->Lp = ceil_div(L, kTrip) * kTrip;
  pl->chained = chained;
  // 32-token blocks (half the barriers, all of the LDS) where every
  // workgroup of the readout scan has a CU to itself.
  const bool tb32_ok = variant_has_tb32(npl, G, vw, kModeFull);
  pl->tb = (tb32_ok && (chained || (n_long == T && T <= kNumCU))) ? 32 : 16;
  const char* te = getenv("SSM_SCAN_TB");
  if (te && tb32_ok && (atoi(te) == 16 || atoi(te) == 32)) pl->tb = atoi(te);
  pl->packed = false;
  pl->trap = rule == kRuleTrap;
  pl->direct = direct;
}

// Packed sequences (batch row 0 holds nseq of them): every (tile column,
// sequence) is one readout-pass unit from its own initial state, with no
// chunking of a sequence.
void plan_packed(int64_t L, int64_t dim, int64_t N, int64_t es, int vw_ok, int64_t nseq, int rule, Plan* pl) {
  const int64_t kNumCU = device_cu_count();
  int npl, G;
  if (N == 16) {
    npl = 2;
    G = 8;
  } else {
    generic_variant(N, &npl, &G);
  }
  pl->npl = npl;
  pl->G = G;
  pl->vw = preferred_vw(G) <= vw_ok ? preferred_vw(G) : 1;
  pl->ntd = static_cast<int>(ceil_div(dim, 64));
  pl->n_long = 0;
  pl->n_split = pl->ntd;
  pl->Ks = static_cast<int>(nseq);
  pl->chunk_len = L;
  pl->Lp = ceil_div(L, kTrip) * kTrip;
  pl->chained = false;
  pl->packed = true;
  pl->trap = rule == kRuleTrap;
  pl->direct = es == 4 && rule == kRuleEuler;
  const bool tb32_ok = variant_has_tb32(npl, G, pl->vw, kModeFull);
  pl->tb = (tb32_ok && static_cast<int64_t>(pl->ntd) * nseq <= kNumCU) ? 32 : 16;
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

// Zeroes the header words (status, tickets) and ready flags of a call whose
// B and C need no packing (pack_bc_kernel zeroes them otherwise).
__global__ void __launch_bounds__(256) zero_words_kernel(unsigned* words, int n) {
  for (int e = threadIdx.x; e < n; e += 256) words[e] = 0u;
}

template <class IO, int RULE>
hipError_t run_scan(const Plan& pl, const Layout& lay, const void* B, const void* C, float* bc, ScanParams p,
                    hipStream_t s) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.G;
  const dim3 pgrid(static_cast<unsigned>(p.batch * (pl.Lp / kPackT)));
#define SSM_PACK_CASE(NPL_)                                                                                  \
  if (pl.npl == NPL_)                                                                                       \
    hipLaunchKernelGGL((pack_bc_kernel<IO, NPL_>), pgrid, dim3(256), 0, s, B, C, bc, p.batch, p.L, pl.Lp, p.N, \
                       pl.G, p.status, lay.n_words, const_cast<float*>(p.cb));
  if (pl.direct) {
    // the scan reads B and C itself: only the header words and flags need zeroing
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, s, p.status, lay.n_words);
  } else {
    SSM_PACK_CASE(1)
    SSM_PACK_CASE(2)
    SSM_PACK_CASE(4)
    SSM_PACK_CASE(8)
    SSM_PACK_CASE(16)
  }
#undef SSM_PACK_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.order) {
    hipLaunchKernelGGL(packed_order_kernel, dim3(1), dim3(kOrderBins), 0, s, p.cu, pl.Ks, p.L,
                       const_cast<int*>(p.order));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid_full(static_cast<unsigned>(pl.n_long + static_cast<int64_t>(pl.n_split) * pl.Ks));
  if (pl.chained)  // one workgroup per whole tile, each also running at most one chunk
    return launch_scan<IO, kModeChained, RULE>(pl.npl, pl.G, pl.vw, pl.tb, p, dim3(pl.n_long), s);
  if (pl.n_split > 0 && pl.Ks > 1 && !pl.packed) {
    const dim3 grid_agg(static_cast<unsigned>(static_cast<int64_t>(pl.n_split) * (pl.Ks - 1)));
    e = launch_scan<IO, kModeAgg, RULE>(pl.npl, pl.G, pl.vw, 16, p, grid_agg, s);
    if (e != hipSuccess) return e;
    const int64_t cols = static_cast<int64_t>(pl.n_split) * 64 * npad;
    hipLaunchKernelGGL(carry_kernel<kCarryRuns>, dim3(static_cast<unsigned>(ceil_div(cols, kCarryCols))), dim3(256),
                       0, s, static_cast<const float*>(p.aggP), static_cast<const float*>(p.aggS), p.carry,
                       static_cast<int64_t>(pl.n_split), pl.Ks, npad, p.h0, static_cast<int64_t>(pl.n_long),
                       static_cast<int64_t>(pl.ntd), p.dim, p.N);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_scan<IO, kModeFull, RULE>(pl.npl, pl.G, pl.vw, pl.tb, p, grid_full, s);
}

// The decode step keeps no per-channel state across lanes beyond one
// wavefront: 64 lanes of 4 states.
constexpr int64_t kMaxDecodeDstate = 256;

template <class IO>
hipError_t run_decode(const DecodeParams& p, hipStream_t s) {
  const int nq = next_pow2(ceil_div(p.N, 4));
  const size_t es = __is_same(IO, F32) ? 4 : 2;
  const bool vec4 = (p.N % 4) == 0 && aligned(p.state, 16) && aligned(p.A, 16);
  if (vec4 && aligned(p.B, 4 * es) && aligned(p.C, 4 * es)) {
    // R batch rows per thread: A, bias and D are then read once per R rows.
    // Two rows beat four on the 256 x 5120 x 16 step (41 against 49 us from
    // HBM, 33 against 34 us from the Infinity Cache): at four the kernel holds
    // 88 registers, five wavefronts per SIMD, too few loads in flight.
    const int R = p.batch >= 2 ? 2 : 1;
    const int64_t threads = ceil_div(p.batch, R) * p.dim * nq;
    const dim3 grid(static_cast<unsigned>(ceil_div(threads, 256)));
#define SSM_DECV_CASE(NQ_)                                                                         \
  if (nq == NQ_) {                                                                                 \
    if (R == 2)                                                                                    \
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
    SSM_DECV_CASE(32)
    SSM_DECV_CASE(64)
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
  SSM_DEC_CASE(32)
  SSM_DEC_CASE(64)
#undef SSM_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace ssm

using namespace ssm;

namespace ssm {
namespace {

// Workspace of a forward call (nseq > 0: packed sequences; trap: the
// trapezoidal rule).  The layout depends only on the variant, which the
// pointers do not change; size it for the widest and the narrowest prologue
// anyway.  0 for arguments the call would reject.
size_t fwd_workspace(int64_t batch, int64_t L, int64_t dim, int64_t dstate, int64_t nseq, ssm_dtype_t dt,
                     bool trap) {
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > 64 || batch > kMaxBatch) return 0;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return 0;
  const int64_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  const int rule = trap ? kRuleTrap : kRuleEuler;
  const int64_t row = token_row_bytes(dim, dstate, es, es == 4 && !trap);
  Plan p4, p1;
  if (nseq > 0) {
    if (batch != 1 || max_chunk_len(row) < ceil_div(L, kChunkQuantum) * kChunkQuantum) return 0;
    plan_packed(L, dim, dstate, es, 4, nseq, rule, &p4);
    plan_packed(L, dim, dstate, es, 1, nseq, rule, &p1);
  } else {
    if (max_chunk_len(row) < kChunkQuantum) return 0;
    plan_scan(batch, L, dim, dstate, es, 4, rule, &p4);
    plan_scan(batch, L, dim, dstate, es, 1, rule, &p1);
  }
  const size_t a = layout_for(p4, batch).total, b = layout_for(p1, batch).total;
  return a > b ? a : b;
}

// The forward, from given initial states and over packed sequences when
// asked (cu_seqlens non-null: batch 1, nseq sequences).
ssm_status_t scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, int softplus_flag,
                           const float* h0, const int64_t* cu_seqlens, int64_t nseq, void* y, float* final_state,
                           int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt, void* workspace,
                           size_t workspace_bytes, hipStream_t stream, int rule) {
  const ssm_status_t st =
      check_scan_args(u, delta, A, B, C, D, z, delta_bias, y, final_state, batch, L, dim, dstate, dt);
  if (st != SSM_OK) return st;
  if (h0 && !aligned(h0, 4)) return SSM_ERR_INVALID_ARG;
  if (cu_seqlens && (!aligned(cu_seqlens, 8) || batch != 1 || nseq <= 0)) return SSM_ERR_INVALID_ARG;
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
  const int64_t row = token_row_bytes(dim, dstate, static_cast<int64_t>(es), es == 4 && rule == kRuleEuler);
  if (max_chunk_len(row) < kChunkQuantum) return SSM_ERR_UNSUPPORTED;
  Plan pl;
  if (cu_seqlens) {
    // a sequence is never cut, so the whole row of tokens must stay within the 32-bit offsets
    if (ceil_div(L, kChunkQuantum) * kChunkQuantum > max_chunk_len(row)) return SSM_ERR_UNSUPPORTED;
    plan_packed(L, dim, dstate, static_cast<int64_t>(es), vw_ok, nseq, rule, &pl);
  } else {
    plan_scan(batch, L, dim, dstate, static_cast<int64_t>(es), vw_ok, rule, &pl);
  }
  if (static_cast<int64_t>(pl.n_long) + static_cast<int64_t>(pl.n_split) * pl.Ks > 0x7fffffffLL ||
      batch * (pl.Lp / kPackT) > 0x7fffffffLL)
    return SSM_ERR_UNSUPPORTED;
  const Layout lay = layout_for(pl, batch);
  if (!workspace || workspace_bytes < lay.total || !aligned(workspace, 256)) return SSM_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  unsigned* words = reinterpret_cast<unsigned*>(ws);
  ScanParams p = {};
  p.u = u;
  p.delta = delta;
  p.A = A;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.bc = reinterpret_cast<const float*>(ws + lay.words);
  p.Braw = B;
  p.Craw = C;
  p.y = y;
  p.final_state = final_state;
  p.aggP = p.aggS = p.carry = nullptr;
  p.status = words + kWordStatus;
  p.ticket = words + kWordTicket;
  p.flags = pl.chained ? words + kHeaderWords : nullptr;  // [n_split][Ks]
  p.spin_limit = wait_spin_limit();
  p.wait_override = wait_override(words);
  p.h0 = h0;
  p.cu = cu_seqlens;
  size_t off = lay.words + lay.bc;
  if (lay.pairs) {
    p.aggP = reinterpret_cast<float*>(ws + off);
    p.aggS = reinterpret_cast<float*>(ws + off + lay.pairs);
    off += 2 * lay.pairs;
  }
  if (lay.carry) {
    p.carry = reinterpret_cast<float*>(ws + off);
    off += lay.carry;
  }
  const char* oe = getenv("SSM_SCAN_ORDER");
  p.order = (lay.order && !(oe && atoi(oe) == 0)) ? reinterpret_cast<const int*>(ws + off) : nullptr;
  off += lay.order;
  p.cb = lay.cb ? reinterpret_cast<const float*>(ws + off) : nullptr;
  p.batch = batch;
  p.L = L;
  p.Lp = pl.Lp;
  p.dim = dim;
  p.N = dstate;
  p.chunk_len = pl.chunk_len;
  p.ntd = pl.ntd;
  p.n_long = pl.n_long;
  p.n_split = pl.n_split;
  p.Ks = pl.Ks;
  p.softplus = softplus_flag ? 1 : 0;
  float* bc = reinterpret_cast<float*>(ws + lay.words);
  hipError_t e;
  if (pl.trap)
    e = dt == SSM_DTYPE_F32 ? run_scan<F32, kRuleTrap>(pl, lay, B, C, bc, p, stream)
                            : run_scan<BF16, kRuleTrap>(pl, lay, B, C, bc, p, stream);
  else
    e = dt == SSM_DTYPE_F32 ? run_scan<F32, kRuleEuler>(pl, lay, B, C, bc, p, stream)
                            : run_scan<BF16, kRuleEuler>(pl, lay, B, C, bc, p, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace
}  // namespace ssm

extern "C" size_t ssm_scan_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt) {
  return fwd_workspace(batch, L, dim, dstate, 0, dt, false);
}

extern "C" ssm_status_t ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                     const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                     void* y, float* final_state, int64_t batch, int64_t L, int64_t dim,
                                     int64_t dstate, ssm_dtype_t dt, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus_flag, nullptr, nullptr, 0, y, final_state,
                       batch, L, dim, dstate, dt, workspace, workspace_bytes, stream, kRuleEuler);
}

extern "C" size_t ssm_scan_fwd_ex_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                                                 int64_t nseq, ssm_dtype_t dt) {
  return fwd_workspace(batch, L, dim, dstate, nseq, dt, false);
}

extern "C" ssm_status_t ssm_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                                        const void* C, const float* D, const void* z, const float* delta_bias,
                                        int softplus_flag, const float* initial_state, const int64_t* cu_seqlens,
                                        int64_t nseq, void* y, float* final_state, int64_t batch, int64_t L,
                                        int64_t dim, int64_t dstate, ssm_dtype_t dt, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state, cu_seqlens,
                       cu_seqlens ? nseq : 0, y, final_state, batch, L, dim, dstate, dt, workspace,
                       workspace_bytes, stream, kRuleEuler);
}

extern "C" size_t ssm_scan_trap_fwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                                                   int64_t nseq, ssm_dtype_t dt) {
  return fwd_workspace(batch, L, dim, dstate, nseq, dt, true);
}

extern "C" ssm_status_t ssm_scan_trap_fwd(const void* u, const void* delta, const float* A, const void* B,
                                          const void* C, const float* D, const void* z, const float* delta_bias,
                                          int softplus_flag, const float* initial_state, const int64_t* cu_seqlens,
                                          int64_t nseq, void* y, float* final_state, int64_t batch, int64_t L,
                                          int64_t dim, int64_t dstate, ssm_dtype_t dt, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state, cu_seqlens,
                       cu_seqlens ? nseq : 0, y, final_state, batch, L, dim, dstate, dt, workspace,
                       workspace_bytes, stream, kRuleTrap);
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
  // up to 64 lanes of 4 states per channel: the whole wavefront for dstate 256
  if (dstate > kMaxDecodeDstate) return SSM_ERR_UNSUPPORTED;
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

// ---- the allocation-free forward
//
// Its workspace is this static device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name stands for a host-side shadow, not device memory, so
// the host never passes it anywhere: scratch_address() looks up each device's
// address once (hipGetSymbolAddress, with that device current) and the calls
// use that.  Every call on a device shares the array; the first kernel of each
// call resets the words that must start at zero (status, ticket, ready
// flags), and everything else is written before it is read.
namespace ssm {

constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// The device address of the current device's array, or null on failure.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace ssm

extern "C" ssm_status_t ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                                             const void* C, const float* D, const void* z, const float* delta_bias,
                                             int softplus_flag, void* y, float* final_state, int64_t batch,
                                             int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                                             hipStream_t stream) {
  const ssm_status_t st =
      check_scan_args(u, delta, A, B, C, D, z, delta_bias, y, final_state, batch, L, dim, dstate, dt);
  if (st != SSM_OK) return st;
  const size_t need = fwd_workspace(batch, L, dim, dstate, 0, dt, false);
  if (need == 0) return SSM_ERR_UNSUPPORTED;      // a shape ssm_scan_fwd rejects as well
  if (need > kScratchBytes) return SSM_ERR_SCRATCH_TOO_SMALL;
  void* ws = scratch_address();
  if (!ws) return SSM_ERR_HIP;
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus_flag, nullptr, nullptr, 0, y, final_state,
                       batch, L, dim, dstate, dt, ws, kScratchBytes, stream, kRuleEuler);
}

// ---- the structured-A forward: one channel per lane (lane_kernels.hpp)
namespace ssm {
namespace {

constexpr int64_t kLaneQuantum = 2 * kLaneTG;  // chunk lengths: whole trips of the main loop (two groups)
constexpr int64_t kLaneMinChunk = 64;          // never cut the sequence finer than this
constexpr int64_t kLaneUnitsPerCU = 10;        // chunk units per CU: about 2.5 wavefronts per SIMD
constexpr int64_t kLaneMaxDstate = 16;         // a lane holds all states of its channel
constexpr int kLaneShortChain = 64;            // carries of at most this many pairs: one thread per column

struct LanePlan {
  int ns;             // states per lane: 4, 8 or 16
  int ntd, n_tiles;   // 64-channel tiles per batch row, in all
  int K;              // chunks per tile
  int64_t chunk_len;
  int64_t Lp;         // token rows of the packed B/C records per batch row
  bool packed_bc;     // bf16 storage: B and C packed into fp32 records first
};

struct LaneLayout {
  size_t words, bc, pairs, total;
};

// A tile (64 channels of one batch row) is one wavefront, so every tile is cut
// into K chunks.  The passes are issue-bound and their units are equal, so a
// pass takes about (units on the busiest SIMD) x (tokens per chunk); K is
// chosen to minimise the pair pass (about 0.56 of a full-pass token each, one
// unit fewer per tile) plus the full pass plus the carry's memory traffic,
// with a single wavefront on a SIMD counted at 0.7 of the issue rate, chunks
// of at least kLaneMinChunk tokens and chunk rows within 32-bit byte offsets.
// SSM_LANE_K (environment) overrides K for tuning sweeps and tests.
double lane_pass_cost(int64_t units, int64_t simds, int64_t chunk) {
  if (units <= 0) return 0.0;
  const int64_t w = ceil_div(units, simds);
  return static_cast<double>(w * chunk) / (w >= 2 ? 1.0 : 0.7);
}

bool plan_lane(int64_t batch, int64_t L, int64_t dim, int64_t N, int64_t es, LanePlan* pl) {
  pl->ns = N <= 4 ? 4 : (N <= 8 ? 8 : 16);
  pl->ntd = static_cast<int>(ceil_div(dim, 64));
  const int64_t T = batch * pl->ntd;
  if (T > 0x7fffffffLL) return false;
  pl->n_tiles = static_cast<int>(T);
  // a chunk and the padding of its last trip within 2^31 bytes of token rows (and, read directly, of B rows)
  const int64_t row = (es == 4 && N * 4 > dim * es) ? N * 4 : dim * es;
  const int64_t cmax = (0x7fffffffLL / row - 2 * kLaneQuantum) / kLaneQuantum * kLaneQuantum;
  if (cmax < kLaneQuantum) return false;
  const int64_t simds = 4 * device_cu_count();
  int64_t kmax = ceil_div(L, kLaneMinChunk) < kMaxChunks ? ceil_div(L, kLaneMinChunk) : kMaxChunks;
  const int64_t kmin = ceil_div(L, cmax);
  if (kmax < kmin) kmax = kmin;
  // about 0.18 us per full-pass token of one wavefront; the carry moves 3 floats per (chunk, lane, state)
  constexpr double kUsPerToken = 0.18, kBytesPerUs = 5.0e6, kCarryLaunchUs = 4.0;
  int64_t best_k = kmin;
  double best = -1.0;
  for (int64_t K = kmin; K <= kmax; ++K) {
    const int64_t chunk = ceil_div(ceil_div(L, K), kLaneQuantum) * kLaneQuantum;
    if (chunk > cmax || ceil_div(L, chunk) != K) continue;
    double cost = lane_pass_cost(T * K, simds, chunk) + 0.56 * lane_pass_cost(T * (K - 1), simds, chunk);
    if (K > 1) cost += (12.0 * T * K * 64 * pl->ns / kBytesPerUs + kCarryLaunchUs) / kUsPerToken;
    if (best < 0.0 || cost < best) {
      best = cost;
      best_k = K;
    }
  }
  int64_t K = best_k;
  const char* ke = getenv("SSM_LANE_K");
  if (ke && atoi(ke) > 0) K = atoi(ke) < kmin ? kmin : atoi(ke);
  if (K > kMaxChunks) K = kMaxChunks;
  int64_t chunk = ceil_div(ceil_div(L, K), kLaneQuantum) * kLaneQuantum;
  if (chunk > cmax) chunk = cmax;
  K = ceil_div(L, chunk);
  if (K > kMaxChunks || T * K > 0x7fffffffLL) return false;
  pl->K = static_cast<int>(K);
  pl->chunk_len = chunk;
  pl->Lp = ceil_div(L, kTrip) * kTrip;
  pl->packed_bc = es == 2;
  return true;
}

LaneLayout lane_layout(const LanePlan& pl, int64_t batch) {
  LaneLayout l;
  l.words = align256(static_cast<size_t>(kHeaderWords) * sizeof(unsigned));
  l.bc = pl.packed_bc ? align256((static_cast<size_t>(batch) * pl.Lp + kTBMax) * 32 * sizeof(float)) : 0;
  l.pairs = pl.K > 1 ? align256(static_cast<size_t>(pl.n_tiles) * pl.K * 64 * pl.ns * sizeof(float)) : 0;
  l.total = l.words + l.bc + 3 * l.pairs;  // chunk fades P, chunk states S, carried-in states
  return l;
}

size_t structured_workspace(int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt) {
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > kLaneMaxDstate || batch > kMaxBatch) return 0;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return 0;
  LanePlan pl;
  if (!plan_lane(batch, L, dim, dstate, dt == SSM_DTYPE_F32 ? 4 : 2, &pl)) return 0;
  return lane_layout(pl, batch).total;
}

template <class IO>
hipError_t run_lane(const LanePlan& pl, const LaneLayout& lay, unsigned* words, const LaneParams& p, hipStream_t s) {
  if (pl.packed_bc) {
    // fp32 records of 16 states (zero past dstate): B_t then C_t; also zeroes the header words
    const dim3 pgrid(static_cast<unsigned>(p.batch * (pl.Lp / kPackT)));
    hipLaunchKernelGGL((pack_bc_kernel<IO, 16>), pgrid, dim3(256), 0, s, p.Braw, p.Craw, const_cast<float*>(p.bc),
                       p.batch, p.L, pl.Lp, p.N, 1, words, kHeaderWords, static_cast<float*>(nullptr));
  } else {
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, s, words, kHeaderWords);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.K > 1) {
    e = launch_lane<IO>(pl.ns, true, false, p, s);
    if (e != hipSuccess) return e;
    // short chains: one thread walks a whole column; long ones are cut into runs
    const int64_t cols = static_cast<int64_t>(pl.n_tiles) * 64 * pl.ns;
    const bool one = pl.K - 1 <= kLaneShortChain;
    const dim3 cgrid(static_cast<unsigned>(ceil_div(cols, one ? 256 : kCarryCols)));
    if (one)
      hipLaunchKernelGGL(carry_kernel<1>, cgrid, dim3(256), 0, s, static_cast<const float*>(p.aggP),
                         static_cast<const float*>(p.aggS), p.carry, static_cast<int64_t>(pl.n_tiles), pl.K,
                         static_cast<int64_t>(pl.ns), p.h0, static_cast<int64_t>(0), static_cast<int64_t>(pl.ntd),
                         p.dim, p.N);
    else
      hipLaunchKernelGGL(carry_kernel<kCarryRuns>, cgrid, dim3(256), 0, s, static_cast<const float*>(p.aggP),
                         static_cast<const float*>(p.aggS), p.carry, static_cast<int64_t>(pl.n_tiles), pl.K,
                         static_cast<int64_t>(pl.ns), p.h0, static_cast<int64_t>(0), static_cast<int64_t>(pl.ntd),
                         p.dim, p.N);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_lane<IO>(pl.ns, true, true, p, s);
}

}  // namespace
}  // namespace ssm

extern "C" size_t ssm_scan_fwd_structured_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                                                         ssm_dtype_t dt) {
  return structured_workspace(batch, L, dim, dstate, dt);
}

extern "C" ssm_status_t ssm_scan_fwd_structured(const void* u, const void* delta, const float* A0, const void* B,
                                                const void* C, const float* D, const void* z,
                                                const float* delta_bias, int softplus_flag,
                                                const float* initial_state, void* y, float* final_state,
                                                int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                                                ssm_dtype_t dt, void* workspace, size_t workspace_bytes,
                                                hipStream_t stream) {
  const ssm_status_t st =
      check_scan_args(u, delta, A0, B, C, D, z, delta_bias, y, final_state, batch, L, dim, dstate, dt);
  if (st != SSM_OK) return st;
  if (initial_state && !aligned(initial_state, 4)) return SSM_ERR_INVALID_ARG;
  if (dstate > kLaneMaxDstate) return SSM_ERR_UNSUPPORTED;
  const int64_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  LanePlan pl;
  if (!plan_lane(batch, L, dim, dstate, es, &pl)) return SSM_ERR_UNSUPPORTED;
  if (pl.packed_bc && batch * (pl.Lp / kPackT) > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;
  const LaneLayout lay = lane_layout(pl, batch);
  if (!workspace || workspace_bytes < lay.total || !aligned(workspace, 256)) return SSM_ERR_INVALID_ARG;
  char* ws = static_cast<char*>(workspace);
  unsigned* words = reinterpret_cast<unsigned*>(ws);
  LaneParams p = {};
  p.u = u;
  p.delta = delta;
  p.A = A0;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.bc = pl.packed_bc ? reinterpret_cast<const float*>(ws + lay.words) : nullptr;
  p.bc_rows = batch * pl.Lp + kTBMax;
  p.Braw = B;
  p.Craw = C;
  p.y = y;
  p.final_state = final_state;
  p.h0 = initial_state;
  if (lay.pairs) {
    char* pr = ws + lay.words + lay.bc;
    p.aggP = reinterpret_cast<float*>(pr);
    p.aggS = reinterpret_cast<float*>(pr + lay.pairs);
    p.carry = reinterpret_cast<float*>(pr + 2 * lay.pairs);
  }
  p.batch = batch;
  p.L = L;
  p.Lp = pl.Lp;
  p.dim = dim;
  p.N = dstate;
  p.chunk_len = pl.chunk_len;
  p.ntd = pl.ntd;
  p.n_tiles = pl.n_tiles;
  p.K = pl.K;
  p.softplus = softplus_flag ? 1 : 0;
  const hipError_t e = dt == SSM_DTYPE_F32 ? run_lane<F32>(pl, lay, words, p, stream)
                                           : run_lane<BF16>(pl, lay, words, p, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" ssm_status_t ssm_workspace_status(const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || workspace_bytes == 0) return SSM_OK;  // no workspace: no chained plan ran
  if (workspace_bytes < kHeaderWords * sizeof(unsigned) || !aligned(workspace, 256)) return SSM_ERR_INVALID_ARG;
  unsigned status = 0;
  if (hipMemcpyAsync(&status, static_cast<const unsigned*>(workspace) + kWordStatus, sizeof(status),
                     hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SSM_ERR_HIP;
  return (status & kStatusHandoffTimeout) ? SSM_ERR_HANDOFF_TIMEOUT : SSM_OK;
}

extern "C" const char* ssm_status_string(ssm_status_t s) {
  switch (s) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
    case SSM_ERR_HIP: return "SSM_ERR_HIP";
    case SSM_ERR_HANDOFF_TIMEOUT: return "SSM_ERR_HANDOFF_TIMEOUT";
    case SSM_ERR_SCRATCH_TOO_SMALL: return "SSM_ERR_SCRATCH_TOO_SMALL";
  }
  return "SSM_ERR_UNKNOWN";
}
