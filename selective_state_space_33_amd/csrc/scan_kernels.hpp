// scan_kernels.hpp -- gfx950 kernels of the selective scan forward pass.
//
// Work decomposition.  A workgroup owns 64 consecutive channels d of one batch
// row (a "tile") and a stretch of the sequence.  It has G wavefronts;
// wavefront w owns the states n in [w*NPL, (w+1)*NPL) of those 64 channels,
// one channel per lane, so each lane runs NPL independent fp32 recurrences in
// registers, and the B_t, C_t it needs are the same for the whole wavefront.
//
// B and C are first packed (pack_bc_kernel) into fp32 records per state group,
//   bc[b][g][t][0 .. NPL)       = B_t[g*NPL .. g*NPL+NPL)
//   bc[b][g][t][NPL .. 2*NPL)   = C_t[g*NPL .. g*NPL+NPL)
// (states beyond dstate are zero), so a wavefront fetches the B_t/C_t of
// several tokens with one 64-byte scalar load and uses them as SGPR operands,
// with no per-token conversion work.
//
// The sequence is processed in blocks of TB tokens, software-pipelined over
// three blocks with double-buffered LDS and one barrier per block: while the
// wavefronts scan block k they also
//   - (epilogue of block k-1) sum the G partial readouts of each (token,
//     channel) in a fixed order, add D*u, multiply by SiLU(z), round, store y;
//   - (prologue of block k+1) turn the u, delta_raw, z loaded two blocks
//     earlier (coalesced buffer loads) into delta = softplus(raw + bias) and
//     delta*u, once per (token, channel), staged in LDS;
//   - issue the loads of block k+3.
// The main loop has no data-dependent branch: the sequence is padded to whole
// trips of blocks, token rows past the end read as zero through the buffer
// resources' range check (and their stores are dropped), and a padding
// token's delta is forced to 0, which makes its step the identity pair (1, 0).
// The scan of block k walks its TB tokens: for every state
// a = exp2(delta * A*log2 e), h = a*h + (delta*u)*B_t[n], and the partial
// readout y_w = sum over its states of C_t[n]*h -- the fade-and-add pair
// (a, b) of each step never leaves registers.  The packed B/C records and the
// staged (delta, delta*u) of the next group of tokens are fetched while the
// current group is computed.
//
// Tiles are either scanned whole by one workgroup ("long" tiles) or, when
// there are too few tiles to fill the GPU evenly, cut into Ks chunks of the
// sequence ("Mamba is attention all you really need, part 2", "The relay":
// squash each chunk into one fade-and-add pair, combine the chunk pairs, pass
// the real states back):
//   aggregate (FULL = false) scans chunks 0..Ks-2 of every split tile from a
//             zero state and writes each chunk's pair (P, S) per (d, n): S is
//             the state the chunk reaches from zero, P = exp(A * sum of its
//             deltas) its total fade;
//   carry     composes the pairs in order and writes the state entering every
//             chunk;
//   scan (FULL = true) runs the long tiles whole and every chunk of the split
//             tiles from its carried-in state, producing y and the final state.
#pragma once

#include <utility>

#include "common.hpp"

namespace ssm {

struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  const float* bc;     // packed B/C records [batch][G][Lp][2*NPL]
  void* y;
  float* final_state;  // nullable
  // Chunk pairs and carried-in states of the split tiles: [n_split][Ks][64][Npad].
  float* aggP;
  float* aggS;
  float* carry;
  int64_t batch, L, Lp, dim, N;
  int64_t chunk_len;   // tokens per chunk of a split tile
  int ntd;             // 64-channel tiles per batch row
  int n_long;          // tiles 0 .. n_long-1 are scanned whole
  int Ks;              // chunks per split tile (tiles n_long .. T-1)
  int softplus;
};

// Tokens per staged block (every variant), and the prologue layout: a thread
// handles VW consecutive channels of RPT token rows.
constexpr int kTB = 16;
template <int G, int VW> struct BlockShape {
  static constexpr int TB = kTB;
  static_assert(G * VW <= kTB, "a block row must fit the prologue threads");
  static constexpr int RPT = TB / (G * VW);
};

// Tokens per group: one group's packed B/C records are 16 floats (32 for NPL 16).
template <int NPL> struct GroupShape {
  static constexpr int SUB = (NPL >= 8) ? 1 : 8 / NPL;
  static constexpr int FLOATS = SUB * 2 * NPL;
  static constexpr int VEC16 = FLOATS / 16;
  static_assert(FLOATS % 16 == 0, "group records are whole 16-float loads");
};

template <int I> struct IC { static constexpr int value = I; };

// Ring of raw token blocks (u, delta_raw, z) in registers.  Block k+kPD+1 is
// loaded while block k is scanned, staged by the prologue while block k+kPD is
// scanned, and its u, z are read again by its epilogue while block k+kPD+2 is
// scanned, so the ring has kRing = kPD + 2 slots and the main loop is unrolled
// by kRing:
// every slot is then written and read at fixed points of the loop body and
// stays in the same registers across iterations (no copies, so no waits on
// loads in flight).
constexpr int kPD = 2;
constexpr int kRing = kPD + 2;
// Tokens per unrolled trip of the main loop.  Chunk lengths and the packed B/C
// rows are multiples of it; one group of records past the end is read (and
// not used), so the packed buffer carries kTB rows of padding.
constexpr int kTrip = kRing * kTB;

// lgkmcnt(0) with vmcnt and expcnt left at their maxima (gfx9 encoding).
constexpr int kWaitLgkm0 = 0xC07F;

// Pack B and C ([batch][L][N], fp32 or bf16) into fp32 per-group records
// [batch][G][Lp][2*NPL]; states n >= N and tokens t >= L are zero.  A
// workgroup transposes kPackT tokens through LDS: the token rows are read
// contiguously (one element per thread), the records written contiguously
// (one record per thread, vector stores).
constexpr int kPackT = 16;

template <class IO, int NPL>
__global__ void __launch_bounds__(256) pack_bc_kernel(const void* __restrict__ B, const void* __restrict__ C,
                                                     float* __restrict__ bc, int64_t batch, int64_t L, int64_t Lp,
                                                     int64_t N, int G) {
  __shared__ float sB[kPackT * 64], sC[kPackT * 64];
  const int Npad = NPL * G;  // <= 64
  const int64_t nblk = Lp / kPackT;
  const int64_t b = blockIdx.x / nblk;
  const int64_t t0 = (blockIdx.x % nblk) * kPackT;
  for (int e = threadIdx.x; e < kPackT * Npad; e += 256) {
    const int tt = e / Npad, n = e % Npad;
    const int64_t t = t0 + tt;
    const bool ok = t < L && n < N;
    sB[e] = ok ? load_elem<IO>(B, (b * L + t) * N + n) : 0.0f;
    sC[e] = ok ? load_elem<IO>(C, (b * L + t) * N + n) : 0.0f;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < G * kPackT; q += 256) {
    const int g = q / kPackT, tt = q % kPackT;
    float rec[2 * NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      rec[j] = sB[tt * Npad + g * NPL + j];
      rec[NPL + j] = sC[tt * Npad + g * NPL + j];
    }
    float* out = bc + ((b * G + g) * Lp + t0 + tt) * (2 * NPL);
    if constexpr (NPL == 1) {
      *reinterpret_cast<float2*>(out) = make_float2(rec[0], rec[1]);
    } else {
#pragma unroll
      for (int v = 0; v < NPL / 2; ++v)
        reinterpret_cast<float4*>(out)[v] = make_float4(rec[4 * v], rec[4 * v + 1], rec[4 * v + 2], rec[4 * v + 3]);
    }
  }
}

// TOUCH: also read one word per 128-byte line of each upcoming block's packed
// B/C records with the vector loads of the ring, so that the wavefronts'
// scalar loads of those records hit in L2.  That pays off when a CU holds a
// single workgroup (latency exposed) or the records stream from HBM (long
// sequences cut into chunks); with two workgroups per CU and L2-resident
// records it only adds issue work, so the planner turns it off there.
template <class IO, int NPL, int G, int VW, bool FULL, bool TOUCH>
__global__ void __launch_bounds__(64 * G) scan_kernel(ScanParams p) {
  constexpr int NPAD = NPL * G;
  constexpr int TB = BlockShape<G, VW>::TB;
  constexpr int RPT = BlockShape<G, VW>::RPT;
  constexpr int RPR = 64 / VW;              // prologue threads per token row
  constexpr int ROWSTEP = (64 * G) / RPR;   // rows between one thread's runs
  static_assert(TB == RPT * ROWSTEP, "block shape");
  using GS = GroupShape<NPL>;
  constexpr int SUB = GS::SUB, NG = TB / SUB;
  static_assert(NG % 2 == 0, "groups come in pairs (double-buffered)");
  static_assert(kRing % 2 == 0, "ring slots keep their block parity");
  constexpr int ES = __is_same(IO, F32) ? 4 : 2;  // bytes per stored element

  // Double-buffered by block parity.
  __shared__ float2 sDU[2][TB][64];                            // (delta, delta*u) per token, channel
  __shared__ float sY[FULL ? 2 : 1][FULL ? G : 1][TB][64];     // partial readouts per wavefront

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t dim = p.dim, L = p.L, N = p.N;

  // ---- which tile and which part of the sequence this workgroup scans
  const int bid = blockIdx.x;
  int tile, c, st;
  bool split;
  if (FULL && bid < p.n_long) {
    tile = bid;
    c = 0;
    st = 0;
    split = false;
  } else {
    const int per = FULL ? p.Ks : p.Ks - 1;
    const int j = FULL ? bid - p.n_long : bid;
    st = j / per;
    c = j % per;
    tile = p.n_long + st;
    split = true;
  }
  const int64_t b = tile / p.ntd;
  const int64_t d0 = static_cast<int64_t>(tile % p.ntd) * 64;
  const int64_t t_begin = split ? static_cast<int64_t>(c) * p.chunk_len : 0;
  const int64_t t_end = split ? ((t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L) : L;
  const int64_t rows = t_end - t_begin;
  const int rows32 = static_cast<int>(rows);
  const int64_t pair_row = (static_cast<int64_t>(st) * p.Ks + c) * 64 + lane;   // row of [n_split][Ks][64]
  // Whole trips of kRing blocks; blocks past the chunk are padding whose
  // tokens are identity steps (delta = 0) and whose outputs fall outside the
  // buffers.
  const int ntrips = static_cast<int>((rows + kTrip - 1) / kTrip);
  const int nblocks = ntrips * kRing;

  // ---- scan lane: channel d, states n0 .. n0+NPL-1
  const int64_t d = d0 + lane;
  const bool dvalid = d < dim;
  const int n0 = w * NPL;
  float A2[NPL], h[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = n0 + j;
    A2[j] = (dvalid && n < N) ? p.A[d * N + n] * kLog2e : 0.0f;
    h[j] = 0.0f;
    if (FULL && split && c > 0 && dvalid) h[j] = p.carry[pair_row * NPAD + n];
  }
  float delta_total = 0.0f;  // chunk sum of delta (aggregate pass)

  // packed B/C records of this wavefront's state group, from the chunk's first token
  const float* bc_row = p.bc + ((b * G + w) * p.Lp + t_begin) * (2 * NPL);

  // ---- prologue / epilogue thread: channels pd .. pd+VW-1, rows prow + i*ROWSTEP of a block
  const int pcol = (tid % RPR) * VW;
  const int prow = tid / RPR;
  const int64_t pd = d0 + pcol;
  const bool pvalid = pd < dim;  // dim is a multiple of VW
  float biasv[VW], Dv[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) {
    biasv[e] = (pvalid && p.bias) ? p.bias[pd + e] : 0.0f;
    Dv[e] = (pvalid && p.D) ? p.D[pd + e] : 0.0f;
  }
  const bool has_z = FULL && p.z != nullptr;
  const bool softplus_on = p.softplus != 0;

  // Token rows of u, delta_raw, z, y are reached through buffer resources
  // covering (b, t_begin, d0) up to the end of the chunk's last row, so rows
  // past the chunk read as zero and are not written.  The host keeps a
  // chunk's rows within 2^31 bytes, so offsets are 32-bit.
  const int row_bytes = static_cast<int>(dim * ES);
  const int blk_bytes = TB * row_bytes;
  const int64_t base_off = ((b * L + t_begin) * dim + d0) * ES;
  const int64_t chunk_bytes = rows * row_bytes - d0 * ES;
  const rsrc_t rs_u = make_rsrc(static_cast<const char*>(p.u) + base_off, chunk_bytes);
  const rsrc_t rs_d = make_rsrc(static_cast<const char*>(p.delta) + base_off, chunk_bytes);
  const rsrc_t rs_z = make_rsrc(has_z ? static_cast<const char*>(p.z) + base_off : nullptr, has_z ? chunk_bytes : 0);
  const rsrc_t rs_y = make_rsrc(FULL ? static_cast<const char*>(p.y) + base_off : nullptr, FULL ? chunk_bytes : 0);
  int voff[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) voff[i] = (prow + i * ROWSTEP) * row_bytes + pcol * ES;

  // Raw u, delta_raw, z of kRing blocks (slot = block % kRing).
  Raw<IO, VW> ru[kRing][RPT], rd[kRing][RPT], rz[kRing][RPT];
  // L2 touch of the wavefront's group records (one float per 128-byte line);
  // the records run on for kTB rows of padding past Lp.
  constexpr int kRecBlk = TB * 2 * NPL;  // record floats per block and group
  float touch[kRing];
  const float* touch_row = bc_row + (lane * 32) % kRecBlk;
  const int64_t touch_lim = (p.Lp - t_begin) * 2 * NPL;

  auto issue_loads = [&](auto slotc, int blk) {
    constexpr int S = decltype(slotc)::value;
    const int bo = blk * blk_bytes;
    if constexpr (TOUCH) {
      const int64_t off = static_cast<int64_t>(blk) * kRecBlk;
      touch[S] = (off + kRecBlk <= touch_lim) ? touch_row[off] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      ru[S][i] = buf_load<IO, VW>(rs_u, voff[i] + bo, 0);
      rd[S][i] = buf_load<IO, VW>(rs_d, voff[i] + bo, 0);
    }
    if (has_z) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) rz[S][i] = buf_load<IO, VW>(rs_z, voff[i] + bo, 0);
    }
  };

  // Stage (delta, delta*u) of block blk (parity P) held in ring slot S.
  auto prologue = [&](auto parc, auto slotc, int blk) {
    constexpr int P = decltype(parc)::value;
    constexpr int S = decltype(slotc)::value;
    // the touched word is not needed; consuming it here (where the slot's
    // loads are complete anyway) keeps the load alive at no cost
    if constexpr (TOUCH) asm volatile("" ::"v"(touch[S]));
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = prow + i * ROWSTEP;
      const bool live = blk * TB + row < rows32;
      float uf[VW], df[VW];
      unpack<IO, VW>(ru[S][i], uf);
      unpack<IO, VW>(rd[S][i], df);
      float2 out[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const float x = df[e] + biasv[e];
        // softplus is evaluated either way and selected, so no branch splits
        // the loop body (the flag is uniform, the select is one v_cndmask)
        float dl = softplus_f(x);
        dl = softplus_on ? dl : x;
        dl = live ? dl : 0.0f;  // padding token: the identity step (1, 0)
        out[e] = make_float2(dl, dl * uf[e]);
      }
      if constexpr (VW == 4) {
        float4* dst = reinterpret_cast<float4*>(&sDU[P][row][pcol]);
        dst[0] = make_float4(out[0].x, out[0].y, out[1].x, out[1].y);
        dst[1] = make_float4(out[2].x, out[2].y, out[3].x, out[3].y);
      } else if constexpr (VW == 2) {
        *reinterpret_cast<float4*>(&sDU[P][row][pcol]) = make_float4(out[0].x, out[0].y, out[1].x, out[1].y);
      } else {
        sDU[P][row][pcol] = out[0];
      }
    }
  };

  // Finish block blk (parity P, ring slot S):
  // y = (sum of partial readouts + D*u) * SiLU(z).
  auto epilogue = [&](auto parc, auto slotc, int blk) {
    if constexpr (FULL) {
      constexpr int P = decltype(parc)::value;
      constexpr int S = decltype(slotc)::value;
      const int bo = blk * blk_bytes;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = prow + i * ROWSTEP;
        // all G partials are read before the (fixed-order) sum
        float part[G][VW];
#pragma unroll
        for (int ww = 0; ww < G; ++ww) {
          if constexpr (VW == 4) {
            const float4 v = *reinterpret_cast<const float4*>(&sY[P][ww][row][pcol]);
            part[ww][0] = v.x; part[ww][1] = v.y; part[ww][2] = v.z; part[ww][3] = v.w;
          } else if constexpr (VW == 2) {
            const float2 v = *reinterpret_cast<const float2*>(&sY[P][ww][row][pcol]);
            part[ww][0] = v.x; part[ww][1] = v.y;
          } else {
            part[ww][0] = sY[P][ww][row][pcol];
          }
        }
        float ys[VW];
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          ys[e] = part[0][e];
#pragma unroll
          for (int ww = 1; ww < G; ++ww) ys[e] += part[ww][e];
        }
        float uf[VW], zf[VW], out[VW];
        unpack<IO, VW>(ru[S][i], uf);
        if (has_z) unpack<IO, VW>(rz[S][i], zf);
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          float v = __builtin_fmaf(Dv[e], uf[e], ys[e]);
          if (has_z) v *= silu_f(zf[e]);
          out[e] = v;
        }
        if (pvalid) buf_store<IO, VW>(rs_y, voff[i] + bo, 0, out);
      }
    }
  };

  // One state update for a token: r points at the token's packed record (B then C).
  auto update = [&](auto parc, const float2 dd, const float* r, int tt, float& block_delta) {
    constexpr int P = decltype(parc)::value;
    float yp = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float a = __builtin_amdgcn_exp2f(dd.x * A2[j]);
      h[j] = __builtin_fmaf(a, h[j], dd.y * r[j]);
      if (FULL) yp = __builtin_fmaf(r[NPL + j], h[j], yp);
      // Without the readout store nothing ties the update to its token's
      // group: the optimiser would sink a whole block of updates below all
      // of its record fetches and spill the records.  An empty asm with h as
      // an in/out operand keeps each update where it is written.
      if (!FULL) asm volatile("" : "+v"(h[j]));
    }
    if (FULL) sY[FULL ? P : 0][w][tt][lane] = yp;
    else block_delta += dd.x;
  };

  // Double-buffered group state: packed records (SGPRs) and staged (delta, delta*u).
  float rec[2][GS::FLOATS];
  float2 dd[2][SUB];

  auto fetch_records = [&](auto bufc, int64_t t) {  // t: first token of the group, from t_begin
    constexpr int BUF = decltype(bufc)::value;
    cf32x16_p src = (cf32x16_p)(bc_row + t * (2 * NPL));
#pragma unroll
    for (int v = 0; v < GS::VEC16; ++v) {
      const f32x16_t x = src[v];
#pragma unroll
      for (int k = 0; k < 16; ++k) rec[BUF][16 * v + k] = x[k];
    }
  };
  auto fetch_dd = [&](auto parc, auto bufc, int g) {
    constexpr int P = decltype(parc)::value;
    constexpr int BUF = decltype(bufc)::value;
#pragma unroll
    for (int q = 0; q < SUB; ++q) dd[BUF][q] = sDU[P][g * SUB + q][lane];
  };

  // Group g of the block with parity P from buffer BUF.  The next group's
  // records (the next block's first group after the last one) and staged
  // values are fetched into the other buffer while this one computes.
  auto group = [&](auto parc, auto bufc, auto gc, int64_t t0, float& block_delta) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int g = decltype(gc)::value;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_sched_barrier(0);
    fetch_records(IC<1 - BUF>{}, t0 + (g + 1) * SUB);
    if constexpr (g + 1 < NG) fetch_dd(parc, IC<1 - BUF>{}, g + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < SUB; ++q) update(parc, dd[BUF][q], &rec[BUF][q * 2 * NPL], g * SUB + q, block_delta);
  };

  // Block k (parity P = k % 2, ring slot S = k % kRing): epilogue of k-1,
  // prologue of k+1, loads of k+kPD+1 into the slot block k-1 frees, scan of k.
  auto iteration = [&](auto slotc, int k) {
    constexpr int S = decltype(slotc)::value;
    constexpr int P = S & 1;
    constexpr int Sm1 = (S + kRing - 1) % kRing;  // block k-1, refilled with block k+kPD+1
    constexpr int Sp1 = (S + 1) % kRing;          // block k+1
    static_assert((S + kPD + 1) % kRing == Sm1, "ring");
    IC<P> parc;
    const int64_t t0 = static_cast<int64_t>(k) * TB;
    fetch_dd(parc, IC<0>{}, 0);
    if (k >= 1) epilogue(IC<1 - P>{}, IC<Sm1>{}, k - 1);
    prologue(IC<1 - P>{}, IC<Sp1>{}, k + 1);
    issue_loads(IC<Sm1>{}, k + kPD + 1);
    float block_delta = 0.0f;
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((group(parc, IC<I % 2>{}, IC<I>{}, t0, block_delta)), ...);
    }(std::make_integer_sequence<int, NG>{});
    delta_total += block_delta;
    __syncthreads();
  };

  // fill the ring with blocks 0 .. kPD, stage block 0
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (issue_loads(IC<I>{}, I), ...);
  }(std::make_integer_sequence<int, kPD + 1>{});
  fetch_records(IC<0>{}, 0);
  prologue(IC<0>{}, IC<0>{}, 0);
  __syncthreads();
  for (int k = 0; k < nblocks; k += kRing) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (iteration(IC<I>{}, k + I), ...);
    }(std::make_integer_sequence<int, kRing>{});
  }
  epilogue(IC<1>{}, IC<kRing - 1>{}, nblocks - 1);  // nblocks is a multiple of kRing (even)

  if (!dvalid) return;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = n0 + j;
    if (FULL) {
      if ((!split || c == p.Ks - 1) && p.final_state && n < N) p.final_state[(b * dim + d) * N + n] = h[j];
    } else {
      const int64_t idx = pair_row * NPAD + n;
      p.aggS[idx] = h[j];
      p.aggP[idx] = __builtin_amdgcn_exp2f(A2[j] * delta_total);
    }
  }
}

// State entering each chunk of a split tile: carry_{c+1} = P_c * carry_c + S_c,
// carry_0 = 0, for every column (lane channel, state) of the tile; layout
// [n_split][Ks][64][Npad].  The Ks-1 pairs of a column are cut into kCarryRuns
// runs: each thread composes one run of one column into a single pair, the
// runs' pairs are combined in order through LDS, and each thread walks its
// run again from the state entering it, writing the carries.  A workgroup
// holds kCarryRuns runs of 256 / kCarryRuns columns.
constexpr int kCarryRuns = 32;
constexpr int kCarryCols = 256 / kCarryRuns;

__global__ void __launch_bounds__(256) carry_kernel(const float* __restrict__ P, const float* __restrict__ S,
                                                   float* __restrict__ carry, int64_t n_split, int Ks, int64_t Npad) {
  __shared__ float sP[kCarryRuns][kCarryCols], sS[kCarryRuns][kCarryCols];
  const int run = threadIdx.x / kCarryCols;
  const int cl = threadIdx.x % kCarryCols;
  const int64_t per_tile = 64 * Npad;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * kCarryCols + cl;  // over n_split * per_tile
  const bool ok = col < n_split * per_tile;
  const int64_t st = ok ? col / per_tile : 0, r = col % per_tile;
  const int npairs = Ks - 1;
  const int len = (npairs + kCarryRuns - 1) / kCarryRuns;
  const int c0 = run * len;
  const int c1 = (c0 + len < npairs) ? c0 + len : npairs;
  auto at = [&](int cc) { return (st * Ks + cc) * per_tile + r; };
  // this run's pair: (a, b) composed over chunks c0 .. c1-1, in order
  float a = 1.0f, bb = 0.0f;
  if (ok) {
#pragma unroll 8
    for (int cc = c0; cc < c1; ++cc) {
      const float pc = P[at(cc)];
      a *= pc;
      bb = __builtin_fmaf(pc, bb, S[at(cc)]);
    }
  }
  sP[run][cl] = a;
  sS[run][cl] = bb;
  __syncthreads();
  // state entering this run: the runs before it, composed in order
  float h = 0.0f;
  for (int q = 0; q < run; ++q) h = __builtin_fmaf(sP[q][cl], h, sS[q][cl]);
  if (!ok) return;
#pragma unroll 8
  for (int cc = c0; cc < c1; ++cc) {
    h = __builtin_fmaf(P[at(cc)], h, S[at(cc)]);
    carry[at(cc + 1)] = h;
  }
}

}  // namespace ssm
