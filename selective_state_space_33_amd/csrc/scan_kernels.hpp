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
// When a few tiles more than there are CUs are left over, cutting only those
// into a handful of chunks and running everything in one launch balances the
// GPU better (kModeChained): every chunk workgroup scans its chunk from zero
// (its pair), takes the state carried into it from the chunk before,
// publishes the state it hands on, then runs the full pass, side by side with
// a whole tile on its CU.
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
  // Chained launches: one ready flag per (split tile, chunk), the tickets of
  // whole tiles and of chunks, a status word and the whole tiles running per
  // CU (all zeroed by pack_bc_kernel).
  unsigned* flags;
  unsigned* ticket;      // [0] whole tiles, [1] chunks
  unsigned* status;
  unsigned* cu_whole;    // [kCuSlots]
  int64_t batch, L, Lp, dim, N;
  int64_t chunk_len;   // tokens per chunk of a split tile
  int ntd;             // 64-channel tiles per batch row
  int n_long;          // tiles 0 .. n_long-1 are scanned whole
  int n_split;         // tiles n_long .. n_long+n_split-1 are cut into Ks chunks
  int Ks;              // chunks per split tile
  int softplus;
};

// Launch modes of scan_kernel.
constexpr int kModeFull = 0;     // whole tiles, and chunks of split tiles from their carried-in states
constexpr int kModeAgg = 1;      // chunk pairs (P, S) of chunks 0..Ks-2 of every split tile
constexpr int kModeChained = 2;  // whole tiles and chunk workgroups that chain their carries, in one launch

// A chunk workgroup waits for the state carried into it for at most this many
// polls (each after a short sleep); past that it records an error in the
// status word and goes on from a zero state, so the kernel always ends.
constexpr unsigned kSpinLimit = 1u << 18;
// Slots of the per-CU table: XCC id (4 bits) x the SE/SH/CU bits of HW_ID (8 bits).
constexpr int kCuSlots = 16 * 256;
constexpr unsigned kStatusCarryTimeout = 1u;

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

// lgkmcnt(0) with vmcnt and expcnt left at their maxima, and vmcnt(0) with
// expcnt and lgkmcnt left at theirs (gfx9 s_waitcnt encoding).
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int kWaitVm0 = 0x0F70;

// Pack B and C ([batch][L][N], fp32 or bf16) into fp32 per-group records
// [batch][G][Lp][2*NPL]; states n >= N and tokens t >= L are zero.  A
// workgroup transposes kPackT tokens through LDS: the token rows are read
// contiguously (one element per thread), the records written contiguously
// (one record per thread, vector stores).
constexpr int kPackT = 16;

template <class IO, int NPL>
__global__ void __launch_bounds__(256) pack_bc_kernel(const void* __restrict__ B, const void* __restrict__ C,
                                                     float* __restrict__ bc, int64_t batch, int64_t L, int64_t Lp,
                                                     int64_t N, int G, unsigned* __restrict__ zero_words,
                                                     int n_zero) {
  __shared__ float sB[kPackT * 64], sC[kPackT * 64];
  // the chained scan's flags, ticket and status start at zero on every call
  if (blockIdx.x == 0)
    for (int e = threadIdx.x; e < n_zero; e += 256) zero_words[e] = 0u;
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
// A chained launch must keep two workgroups per CU (a whole tile and a chunk
// workgroup side by side), so its register budget is capped accordingly.
template <class IO, int NPL, int G, int VW, int MODE, bool TOUCH>
__global__ void __launch_bounds__(64 * G, MODE == kModeChained ? 2 : 1) scan_kernel(ScanParams p) {
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
  constexpr bool HAS_FULL = MODE != kModeAgg;      // a full (readout) pass runs in this launch

  // Double-buffered by block parity.
  __shared__ float2 sDU[2][TB][64];                                  // (delta, delta*u) per token, channel
  __shared__ float sY[HAS_FULL ? 2 : 1][HAS_FULL ? G : 1][TB][64];   // partial readouts per wavefront

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t dim = p.dim, L = p.L, N = p.N;

  // ---- which work unit this workgroup runs.  Chained launches number units
  // in the order workgroups start (a ticket), so a chunk only ever waits for
  // a unit that has already started.
  int unit = blockIdx.x;
  if constexpr (MODE == kModeChained) {
    // A workgroup takes a whole tile if none runs on its CU yet, else a chunk
    // (falling back to the other kind when its kind is used up), so each CU
    // pairs one whole tile with chunk work.  Chunks are numbered by a ticket
    // of their own in the order workgroups take them, chunk-major, so a chunk
    // only waits for a chunk that has already started.  The choice goes
    // through the staging buffer, not yet in use (an extra LDS word would
    // push two workgroups past the CU's 160 KB).
    unsigned* sUnit = reinterpret_cast<unsigned*>(&sDU[0][0][0]);
    if (tid == 0) {
      const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID: CU, SH, SE in bits 8..15
      const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
      const unsigned slot = ((xcc & 15u) << 8) | ((hw >> 8) & 255u);
      const unsigned on_cu =
          __hip_atomic_fetch_add(p.cu_whole + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned n_whole = static_cast<unsigned>(p.n_long);
      const unsigned n_chunk = static_cast<unsigned>(p.n_split) * static_cast<unsigned>(p.Ks);
      unsigned kind = on_cu == 0u ? 0u : 1u;
      unsigned u = 0;
      for (int attempt = 0; attempt < 2; ++attempt, kind ^= 1u) {
        const unsigned cap = kind == 0u ? n_whole : n_chunk;
        const unsigned t = __hip_atomic_fetch_add(p.ticket + kind, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t < cap) {
          u = kind == 0u ? t : n_whole + t;
          break;
        }
      }
      *sUnit = u;
    }
    __syncthreads();
    unit = static_cast<int>(__builtin_amdgcn_readfirstlane(*sUnit));
    __syncthreads();  // every wavefront has read it before the buffer is written
  }
  int tile, c, st;
  bool split;
  if (MODE != kModeAgg && unit < p.n_long) {
    tile = unit;
    c = 0;
    st = 0;
    split = false;
  } else if (MODE == kModeChained) {
    // chunk-major: chunk c of every split tile precedes chunk c+1 of any
    const int j = unit - p.n_long;
    c = j / p.n_split;
    st = j % p.n_split;
    tile = p.n_long + st;
    split = true;
  } else {
    const int per = MODE == kModeFull ? p.Ks : p.Ks - 1;
    const int j = MODE == kModeFull ? unit - p.n_long : unit;
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
  }

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
  const bool has_z = HAS_FULL && p.z != nullptr;
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
  const rsrc_t rs_y =
      make_rsrc(HAS_FULL ? static_cast<const char*>(p.y) + base_off : nullptr, HAS_FULL ? chunk_bytes : 0);
  int voff[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) voff[i] = (prow + i * ROWSTEP) * row_bytes + pcol * ES;

  // L2 touch of the wavefront's group records (one float per 128-byte line);
  // the records run on for kTB rows of padding past Lp.
  constexpr int kRecBlk = TB * 2 * NPL;  // record floats per block and group
  const float* touch_row = bc_row + (lane * 32) % kRecBlk;
  const int64_t touch_lim = (p.Lp - t_begin) * 2 * NPL;

  // One pass over the chunk: FULL = true produces y (readout and epilogue),
  // FULL = false only advances h.  Returns the chunk's sum of delta.
  auto run_pass = [&](auto fullc) -> float {
    constexpr bool FULL = decltype(fullc)::value;
    static_assert(!FULL || HAS_FULL, "a readout pass needs the partial-readout buffers");
    float delta_total = 0.0f;

    // Raw u, delta_raw, z of kRing blocks (slot = block % kRing).
    Raw<IO, VW> ru[kRing][RPT], rd[kRing][RPT], rz[kRing][RPT];
    float touch[kRing];

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
      if (FULL && has_z) {
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
      if constexpr (FULL) sY[P][w][tt][lane] = yp;
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
    return delta_total;
  };

  if constexpr (MODE == kModeAgg) {
    // chunk pair from a zero state: S = h, P = exp(A * sum of deltas)
    const float dt = run_pass(IC<false>{});
    if (!dvalid) return;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int64_t idx = pair_row * NPAD + n0 + j;
      p.aggS[idx] = h[j];
      p.aggP[idx] = __builtin_amdgcn_exp2f(A2[j] * dt);
    }
    return;
  } else {
    if (MODE == kModeFull && split && c > 0 && dvalid) {
#pragma unroll
      for (int j = 0; j < NPL; ++j) h[j] = p.carry[pair_row * NPAD + n0 + j];
    }
    if (MODE == kModeChained && split) {
      // Chain the carry: pair of this chunk, state carried in from chunk c-1,
      // state handed on to chunk c+1 (carry row c+1), then the full pass.
      const bool last = c == p.Ks - 1;
      float Pc[NPL], Sc[NPL];
      if (!last) {
        const float dt = run_pass(IC<false>{});
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          Pc[j] = __builtin_amdgcn_exp2f(A2[j] * dt);
          Sc[j] = h[j];
        }
      }
      float cin[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) cin[j] = 0.0f;
      // The carries and flags are read and written only with device-coherent
      // (agent-scope) loads and stores, which bypass the per-XCD L2s; waiting
      // for the carry stores to complete before the flag store orders them.
      // (Release/acquire fences would instead write back or invalidate the
      // whole L2, slowing every workgroup on the XCD.)
      if (c > 0) {
        unsigned* flag = p.flags + static_cast<int64_t>(st) * p.Ks + c;
        if (tid == 0) {
          unsigned polls = 0;
          while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            if (++polls > kSpinLimit) {
              __hip_atomic_fetch_or(p.status, kStatusCarryTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            __builtin_amdgcn_s_sleep(4);
          }
        }
        __syncthreads();
        if (dvalid) {
#pragma unroll
          for (int j = 0; j < NPL; ++j)
            cin[j] = __hip_atomic_load(p.carry + pair_row * NPAD + n0 + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (!last) {
        const int64_t next_row = pair_row + 64;  // carry row of chunk c+1
        if (dvalid) {
#pragma unroll
          for (int j = 0; j < NPL; ++j)
            __hip_atomic_store(p.carry + next_row * NPAD + n0 + j, __builtin_fmaf(Pc[j], cin[j], Sc[j]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this thread's carry stores have completed
        __syncthreads();
        if (tid == 0)
          __hip_atomic_store(p.flags + static_cast<int64_t>(st) * p.Ks + c + 1, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int j = 0; j < NPL; ++j) h[j] = cin[j];
    }
    run_pass(IC<true>{});
    if (!dvalid) return;
    if ((!split || c == p.Ks - 1) && p.final_state) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (n0 + j < N) p.final_state[(b * dim + d) * N + n0 + j] = h[j];
    }
  }
}

}  // namespace ssm
