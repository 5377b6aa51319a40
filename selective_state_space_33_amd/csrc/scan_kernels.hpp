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
// (states beyond dstate are zero).  A wavefront loads a block's records with
// vector loads, 16 consecutive floats per register, each replicated in the
// four 16-lane rows, and an update takes B_t[n], C_t[n] straight from the
// register with a DPP row broadcast: no conversion work and no scalar loads.
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
// (a, b) of each step never leaves registers.  The staged (delta, delta*u) of
// the next group of tokens are read from LDS while the current group is
// computed; the records of block k+1 are loaded while block k is scanned.
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
// When a few tiles more than there are CUs are left over (the 2.8B-shaped
// layer has 320 for 256 CUs), one workgroup per CU runs one tile whole and
// one chunk of a left-over tile spliced into it (kModeChained): chunk c of a
// left-over tile starts from the final state of chunk c-1, which another
// workgroup has scanned by then, so no chunk-pair pass is needed.
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
  const void* Braw;    // the caller's B and C [batch][L][N]: read directly where the records are not packed
  const void* Craw;
  void* y;
  float* final_state;  // nullable
  // Chunk pairs and carried-in states of the split tiles: [n_split][Ks][64][Npad].
  float* aggP;
  float* aggS;
  float* carry;
  // Chained launches: one ready flag per (split tile, chunk), the workgroup
  // ticket and the status word (all zeroed by pack_bc_kernel).  spin_limit
  // bounds each wait; wait_override (a test hook, normally null) is a word no
  // one sets, polled instead of every flag, so every wait runs out.
  unsigned* flags;
  unsigned* ticket;
  unsigned* status;
  unsigned spin_limit;
  const unsigned* wait_override;
  int64_t batch, L, Lp, dim, N;
  int64_t chunk_len;   // tokens per chunk of a split tile
  int ntd;             // 64-channel tiles per batch row
  int n_long;          // tiles 0 .. n_long-1 are scanned whole
  int n_split;         // tiles n_long .. n_long+n_split-1 are cut into Ks chunks
  int Ks;              // chunks per split tile
  int softplus;
  // Checkpoint launches: the state entering every block of every tile,
  // [tiles][ckpt_blocks][64][NPL*G].
  float* ckpt;
  int64_t ckpt_blocks;
  // Initial states h_{-1} [rows][dim][N] (nullable: zero), rows being the
  // batch rows, or the packed sequences when cu is given.  With cu (device
  // offsets, nseq + 1 of them) batch row 0 holds nseq packed sequences: split
  // "chunk" c of a tile column is sequence c, tokens cu[c] .. cu[c+1]-1, with
  // its own initial and final state.
  const float* h0;
  const int64_t* cu;
  // Packed launches: the sequences in launch order (nullable: index order);
  // unit j scans tile column j % n_split of sequence order[j / n_split].
  const int* order;
  // Trapezoidal rule: C_t . B_t per token, [batch][Lp + kTBMax] (pack_bc_kernel).
  const float* cb;
};

// Launch modes of scan_kernel.
constexpr int kModeFull = 0;     // whole tiles, and chunks of split tiles from their carried-in states
constexpr int kModeAgg = 1;      // chunk pairs (P, S) of chunks 0..Ks-2 of every split tile
constexpr int kModeChained = 2;  // one workgroup per CU: a whole tile with one chunk of a left-over tile spliced in
constexpr int kModeCkpt = 3;     // whole tiles, no readout: the state entering every block (for the backward pass)
constexpr int kModeChainedCkpt = 4;  // kModeChained's plan with kModeCkpt's work (no readout, checkpoints)


// Tokens per staged block: 16, or 32 where one workgroup has the CU to
// itself (the block's barrier is then paid half as often, and the staging
// buffers take the whole 160 KB of LDS).  A prologue thread handles VW
// consecutive channels of RPT token rows.
constexpr int kTBMax = 32;
template <int G, int VW, int TB_> struct BlockShape {
  static constexpr int TB = TB_;
  static_assert(TB == 16 || TB == 32, "block length");
  static_assert(G * VW <= TB, "a block row must fit the prologue threads");
  static constexpr int RPT = TB / (G * VW);
};

// Tokens per group: one group's packed B/C records are 16 floats (32 for NPL 16).
template <int NPL> struct GroupShape {
  static constexpr int SUB = (NPL >= 8) ? 1 : 8 / NPL;
  static constexpr int FLOATS = SUB * 2 * NPL;
  static constexpr int VEC16 = FLOATS / 16;
  static_assert(FLOATS % 16 == 0, "group records are whole 16-float loads");
};


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
// Tokens per unrolled trip of the main loop at the longest block.  Chunk
// lengths and the packed B/C rows are multiples of it (so of every variant's
// trip).  A pass loads the records of one block past its end (not used);
// whatever of them lies past the packed buffer reads as zero through the
// buffer resource's range check.
constexpr int kTrip = kRing * kTBMax;

// vmcnt(0) with expcnt and lgkmcnt left at their maxima (gfx9 s_waitcnt encoding).
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
                                                     int n_zero, float* __restrict__ cb) {
  __shared__ float sB[kPackT * 64], sC[kPackT * 64];
  const int Npad = NPL * G;  // <= 64
  if (blockIdx.x == 0) {
    // the chained scan's flags, ticket and status start at zero on every call
    for (int e = threadIdx.x; e < n_zero; e += 256) zero_words[e] = 0u;
    // so do the kTBMax padding records past the last row, which a pass
    // ending past Lp reads (their products with a zero step must stay zero)
    for (int e = threadIdx.x; e < kTBMax * 2 * Npad; e += 256) bc[batch * Lp * 2 * Npad + e] = 0.0f;
  }
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
  // trapezoidal rule: C_t . B_t of every token (in state order)
  if (cb && threadIdx.x < kPackT) {
    float s = 0.0f;
    for (int n = 0; n < Npad; ++n) s = __builtin_fmaf(sC[threadIdx.x * Npad + n], sB[threadIdx.x * Npad + n], s);
    cb[b * (Lp + kTBMax) + t0 + threadIdx.x] = s;
  }
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

template <class IO, int NPL, int G, int VW, int MODE, int TB_, int RULE>
__global__ void __launch_bounds__(64 * G) scan_kernel(ScanParams p) {
  constexpr int NPAD = NPL * G;
  constexpr int TB = BlockShape<G, VW, TB_>::TB;
  constexpr int RPT = BlockShape<G, VW, TB_>::RPT;
  constexpr int TRIP = kRing * TB;          // tokens per unrolled trip of the main loop
  constexpr int RPR = 64 / VW;              // prologue threads per token row
  constexpr int ROWSTEP = (64 * G) / RPR;   // rows between one thread's runs
  static_assert(TB == RPT * ROWSTEP, "block shape");
  using GS = GroupShape<NPL>;
  constexpr int SUB = GS::SUB, NG = TB / SUB;
  static_assert(NG % 2 == 0, "groups come in pairs (double-buffered)");
  static_assert(kRing % 2 == 0, "ring slots keep their block parity");
  constexpr int ES = __is_same(IO, F32) ? 4 : 2;  // bytes per stored element
  constexpr bool HAS_FULL = MODE == kModeFull || MODE == kModeChained;  // a readout pass runs in this launch
  constexpr bool CHAINED = MODE == kModeChained || MODE == kModeChainedCkpt;
  constexpr bool CKPT = MODE == kModeCkpt || MODE == kModeChainedCkpt;
  static_assert(HAS_FULL || G <= TB_, "stop-flag words in the partial-readout buffer");
  constexpr bool TRAP = RULE == kRuleTrap;
  static_assert(!TRAP || MODE != kModeChainedCkpt, "the trapezoidal backward runs without the chained plan");
  // fp32 storage, two-term rule, outside the backward's checkpoint launches:
  // B and C come straight from the caller's rows, B_t[n] at float t*N + n,
  // instead of from packed records.  A block's record registers then hold its
  // B floats (16 per register: 16/NPL tokens of this wavefront's NPL states)
  // followed by its C floats, and need the host to have made N = NPL * G.
  constexpr bool DIRECT = __is_same(IO, F32) && RULE == kRuleEuler && !CKPT;
  // A block's start goes in the loads' scalar offset (SO = the block's byte
  // offset, no vector add per lane) with 16-token blocks, two workgroups per
  // CU.  With 32-token blocks (one workgroup per CU, two wavefronts per SIMD)
  // the lanes add it themselves: measured on the 2.8B and 130M layers, the
  // scalar form ran 1.5-2.5% slower there in spite of 3% fewer VALU
  // instructions, while it gains 3% on the 16-token blocks of the long fp32
  // sequence.
  constexpr bool SO = TB == 16;

  // Double-buffered by block parity.  (delta, delta*u) per token, channel;
  // (delta, u/2) with the trapezoidal rule.
  __shared__ float2 sDU[2][TB][64];
  __shared__ float sY[HAS_FULL ? 2 : 1][HAS_FULL ? G : 1][TB][64];   // partial readouts per wavefront

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t dim = p.dim, L = p.L, N = p.N;
  const int n0 = w * NPL;                 // this wavefront's states n0 .. n0+NPL-1
  const int pcol = (tid % RPR) * VW;      // prologue / epilogue thread: channels pcol .. pcol+VW-1 of the tile,
  const int prow = tid / RPR;             // rows prow + i*ROWSTEP of a block
  int voff_rel[RPT];                      // (in units of token rows and elements; scaled by set_tile)
#pragma unroll
  for (int i = 0; i < RPT; ++i) voff_rel[i] = prow + i * ROWSTEP;
  // delta = fma(sp_k, log1p(e^-|x|), max(x, sp_lo)): softplus(x) when on
  // (sp_k = 1, sp_lo = 0), x itself when off (sp_k = 0, sp_lo = -inf)
  const float sp_k = p.softplus != 0 ? 1.0f : 0.0f;
  const float sp_lo = p.softplus != 0 ? 0.0f : -__builtin_inff();
  const int row_bytes = static_cast<int>(dim * ES);
  const int blk_bytes = TB * row_bytes;

  // ---- the tile (64 channels of one batch row) and stretch of the sequence
  // a pass works on; set_tile points everything at them.
  int64_t b = 0, d0 = 0, d = 0, pd = 0, t_begin = 0;
  int rows32 = 0;
  bool dvalid = false, pvalid = false, has_z = false;
  bool row_start = false;                  // the stretch starts a recurrence (no input before it)
  float A2[NPL], biasv[VW], Dv[VW];
  const float* bc_row = p.bc;
  rsrc_t rs_u, rs_d, rs_z, rs_y, rs_cb;
  int voff[RPT];
  rsrc_t rs_bc;                            // this wavefront's packed B/C records of the stretch
  float* ckpt_row = nullptr;               // checkpoint launches: this lane's states at the stretch's first block
  const int rec_voff = (lane & 15) * 4;    // lane l holds float l % 16 of a group's 16
  // direct B/C: lane l's float of a register is token (l%16)/NPL, state n0 + (l%16)%NPL of its 16/NPL tokens;
  // a state past N gets an offset at or above 2^31, past every resource's range (which the stretch keeps below
  // 2^31 bytes), so it reads zero like a packed record's padding
  rsrc_t rs_B, rs_C;
  const unsigned dir_voff = (n0 + (lane & 15) % NPL < N)
                                ? static_cast<unsigned>((((lane & 15) / NPL) * N + n0 + (lane & 15) % NPL) * 4)
                                : 0x80000000u;

  auto set_tile = [&](int tile, int64_t tb, int64_t te) {
    b = tile / p.ntd;
    d0 = static_cast<int64_t>(tile % p.ntd) * 64;
    t_begin = tb;
    row_start = tb == 0;
    const int64_t rows = te - tb;
    rows32 = static_cast<int>(rows);
    // scan lane: channel d, states n0 .. n0+NPL-1
    d = d0 + lane;
    dvalid = d < dim;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = n0 + j;
      A2[j] = (dvalid && n < N) ? p.A[d * N + n] * kLog2e : 0.0f;
    }
    // packed B/C records of this wavefront's state group, from the stretch's first token
    bc_row = p.bc + ((b * G + w) * p.Lp + t_begin) * (2 * NPL);
    if constexpr (CKPT)  // from the stretch's first block (a chunk starts on a block boundary)
      ckpt_row = p.ckpt + (static_cast<int64_t>(tile) * p.ckpt_blocks * 64 + lane) * NPAD + n0 +
                 (t_begin / TB) * 64 * NPAD;
    // the records run on for kTBMax rows of padding past Lp
    if constexpr (DIRECT) {
      // rows of B and C from the stretch's first token to the end of the batch row (the host keeps the
      // stretch's offsets below 2^31 bytes)
      const int64_t rb = (b * L + t_begin) * N * static_cast<int64_t>(sizeof(float));
      int64_t rbytes = (L - t_begin) * N * static_cast<int64_t>(sizeof(float));
      if (rbytes > 0x7fffffffLL) rbytes = 0x7fffffffLL;
      rs_B = make_rsrc(static_cast<const char*>(p.Braw) + rb, rbytes);
      rs_C = make_rsrc(static_cast<const char*>(p.Craw) + rb, rbytes);
    } else {
      rs_bc = make_rsrc(bc_row, (p.Lp + kTBMax - t_begin) * 2 * NPL * static_cast<int64_t>(sizeof(float)));
    }
    pd = d0 + pcol;
    pvalid = pd < dim;  // dim is a multiple of VW
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      biasv[e] = (pvalid && p.bias) ? p.bias[pd + e] : 0.0f;
      Dv[e] = (pvalid && p.D) ? p.D[pd + e] : 0.0f;
    }
    has_z = HAS_FULL && p.z != nullptr;
    // Token rows of u, delta_raw, z, y are reached through buffer resources
    // covering (b, t_begin, d0) up to the end of the stretch's last row, so
    // rows past it read as zero and are not written.  The host keeps a
    // stretch within 2^31 bytes, so offsets are 32-bit.
    const int64_t base_off = ((b * L + t_begin) * dim + d0) * ES;
    const int64_t bytes = rows * row_bytes - d0 * ES;
    rs_u = make_rsrc(static_cast<const char*>(p.u) + base_off, bytes);
    rs_d = make_rsrc(static_cast<const char*>(p.delta) + base_off, bytes);
    rs_z = make_rsrc(has_z ? static_cast<const char*>(p.z) + base_off : nullptr, has_z ? bytes : 0);
    rs_y = make_rsrc(HAS_FULL ? static_cast<const char*>(p.y) + base_off : nullptr, HAS_FULL ? bytes : 0);
#pragma unroll
    for (int i = 0; i < RPT; ++i) voff[i] = voff_rel[i] * row_bytes + pcol * ES;
    if constexpr (TRAP && HAS_FULL)  // C_t . B_t of the stretch's tokens (zero past the row)
      rs_cb = make_rsrc(p.cb + b * (p.Lp + kTBMax) + t_begin, (L - t_begin) * static_cast<int64_t>(sizeof(float)));
  };
  // blocks of the current stretch, in whole trips of kRing; blocks past the
  // stretch are padding whose tokens are identity steps (delta = 0) and whose
  // outputs fall outside the buffers
  auto stretch_blocks = [&]() { return (rows32 + TRIP - 1) / TRIP * kRing; };

  float h[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) h[j] = 0.0f;

  // One pass over blocks [k_begin, k_end) of the current stretch (multiples
  // of kRing): FULL = true produces y (readout and epilogue), FULL = false
  // only advances h.  Returns the sum of delta over the blocks.  With a stop
  // flag, the pass also ends after the first trip of kRing blocks that ends
  // at or past block k_stop once the flag is set (k_end then returns the
  // block it stopped at); the flag is polled once per trip, its load in
  // flight while the trip computes.
  // Trapezoidal rule: a pass ends with h, except one stopped by its flag,
  // which leaves the shifted state s for the same workgroup to resume with
  // resume_s = true; that pass re-derives the previous token's step exactly
  // as the prologue did, so a tile split at a point that depends on timing
  // gives the same bits as one pass over it.
  auto run_pass = [&](auto fullc, int k_begin, int& k_end, const unsigned* stop_flag = nullptr,
                      int k_stop = 0, bool resume_s = false) -> float {
    constexpr bool FULL = decltype(fullc)::value;
    static_assert(!FULL || HAS_FULL, "a readout pass needs the partial-readout buffers");
    float delta_total = 0.0f;
    bool stopped = false;
    if (k_begin >= k_end) return delta_total;

    // Raw u, delta_raw, z of kRing blocks (slot = block % kRing).
    Raw<IO, VW> ru[kRing][RPT], rd[kRing][RPT], rz[kRing][RPT];
    // Packed B/C records of two blocks (slot = block parity): register v of a
    // block holds floats 16v .. 16v+15 of its records, float 16v + i in lane i
    // of every 16-lane row, read with row broadcasts.
    constexpr int NRV = TB * 2 * NPL / 16;
    float rv[2][NRV];
    // Trapezoidal rule: C_t . B_t of a prologue thread's rows, per ring slot;
    // the previous token's (delta, u/2) and B (this lane's states) as the
    // scan walks the tokens.
    float rcb[kRing][RPT];
    float pv_d = 0.0f, pv_hx = 0.0f, Bprev[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) Bprev[j] = 0.0f;
    if constexpr (TRAP) {
      // the pass continues a recurrence: token t-1 before its first one is real input
      const int prev_row = k_begin * TB - 1;  // relative to the stretch
      if (!(row_start && k_begin == 0) && t_begin + prev_row >= 0 && prev_row < rows32) {
        if (dvalid) pv_hx = 0.5f * load_elem<IO>(p.u, (b * L + t_begin + prev_row) * dim + d);
        if (resume_s && dvalid)  // h holds s: the previous token's step, as the prologue computed it
          pv_d = step_of(load_elem<IO>(p.delta, (b * L + t_begin + prev_row) * dim + d) +
                             (p.bias ? p.bias[d] : 0.0f), sp_k, sp_lo);
#pragma unroll
        for (int j = 0; j < NPL; ++j) Bprev[j] = bc_row[static_cast<int64_t>(prev_row) * (2 * NPL) + j];
      }
    }

    auto load_records = [&](auto parc, int blk) {
      constexpr int P = decltype(parc)::value;
      if constexpr (DIRECT) {
        const int bo = blk * TB * static_cast<int>(N) * 4;
        const unsigned rstep = (16 / NPL) * static_cast<unsigned>(N) * 4u;  // bytes of B per register
#pragma unroll
        for (int v = 0; v < NRV / 2; ++v) {
          const int off = static_cast<int>(dir_voff + v * rstep) + (SO ? 0 : bo);
          rv[P][v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_B, off, SO ? bo : 0, 0));
          rv[P][NRV / 2 + v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_C, off, SO ? bo : 0, 0));
        }
      } else {
        const int bo = blk * (TB * 2 * NPL * 4);
#pragma unroll
        for (int v = 0; v < NRV; ++v)
          rv[P][v] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs_bc, rec_voff + v * 64 + (SO ? 0 : bo), SO ? bo : 0, 0));
      }
    };
    // float index within a block's records of B_t[n0 + j] and C_t[n0 + j], t = token q of the block
    auto bidx = [](int q, int j) constexpr { return DIRECT ? q * NPL + j : q * 2 * NPL + j; };
    auto cidx = [](int q, int j) constexpr { return DIRECT ? TB * NPL + q * NPL + j : q * 2 * NPL + NPL + j; };

    auto issue_loads = [&](auto slotc, int blk) {
      constexpr int S = decltype(slotc)::value;
      const int bo = blk * blk_bytes;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        ru[S][i] = buf_load<IO, VW>(rs_u, voff[i] + (SO ? 0 : bo), SO ? bo : 0);
        rd[S][i] = buf_load<IO, VW>(rs_d, voff[i] + (SO ? 0 : bo), SO ? bo : 0);
      }
      if (FULL && has_z) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) rz[S][i] = buf_load<IO, VW>(rs_z, voff[i] + (SO ? 0 : bo), SO ? bo : 0);
      }
      if constexpr (TRAP && FULL) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
          rcb[S][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rs_cb, voff_rel[i] * 4 + (SO ? 0 : blk * TB * 4), SO ? blk * TB * 4 : 0, 0));
      }
    };

    // Stage (delta, delta*u) of block blk (parity P) held in ring slot S.
    auto prologue = [&](auto parc, auto slotc, int blk) {
      constexpr int P = decltype(parc)::value;
      constexpr int S = decltype(slotc)::value;
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
          // evaluated either way, so no branch splits the loop body
          float dl = step_of(df[e] + biasv[e], sp_k, sp_lo);
          dl = live ? dl : 0.0f;  // padding token: the identity step (1, 0)
          if constexpr (TRAP) out[e] = make_float2(dl, live ? 0.5f * uf[e] : 0.0f);
          else out[e] = make_float2(dl, dl * uf[e]);
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
          if constexpr (TRAP) {
            // + delta_t (u_t/2) (C_t . B_t): the part of h_t the scan leaves out (see update)
            float st[2 * VW];
            if constexpr (VW == 4) {
              const float4 v0 = *reinterpret_cast<const float4*>(&sDU[P][row][pcol]);
              const float4 v1 = *reinterpret_cast<const float4*>(&sDU[P][row][pcol + 2]);
              st[0] = v0.x; st[1] = v0.y; st[2] = v0.z; st[3] = v0.w;
              st[4] = v1.x; st[5] = v1.y; st[6] = v1.z; st[7] = v1.w;
            } else if constexpr (VW == 2) {
              const float4 v0 = *reinterpret_cast<const float4*>(&sDU[P][row][pcol]);
              st[0] = v0.x; st[1] = v0.y; st[2] = v0.z; st[3] = v0.w;
            } else {
              const float2 v0 = sDU[P][row][pcol];
              st[0] = v0.x; st[1] = v0.y;
            }
#pragma unroll
            for (int e = 0; e < VW; ++e) ys[e] = __builtin_fmaf(st[2 * e] * st[2 * e + 1], rcb[S][i], ys[e]);
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
          if (pvalid) buf_store<IO, VW>(rs_y, voff[i] + (SO ? 0 : bo), SO ? bo : 0, out);
        }
      }
    };

    // The state updates of token q of group g of a block whose records are in
    // slot P: its record (B then C) is floats F .. F + 2*NPL of the block's.
    //
    // Trapezoidal rule.  The recurrence h_t = a_t h_{t-1} + (delta_t/2) a_t
    // B_{t-1} u_{t-1} + (delta_t/2) B_t u_t (a_t = exp(delta_t A)) is scanned as
    //   s_t = h_t - (delta_t/2) B_t u_t
    //       = a_t (s_{t-1} + (delta_{t-1} + delta_t) (u_{t-1}/2) B_{t-1}),
    // which costs an update what the two-term rule does: one fma on the
    // previous token's B (a row broadcast of the record before this one), one
    // multiply by the fade.  The epilogue adds the left-out part of y_t,
    // delta_t (u_t/2) (C_t . B_t), and a pass hands on h (see run_pass's end).
    auto update = [&](auto parc, auto gc, auto qc, const float2 dd, float& block_delta) {
      constexpr int P = decltype(parc)::value;
      constexpr int TQ = decltype(gc)::value * SUB + decltype(qc)::value;  // token within the block
      float yp = 0.0f;
      if constexpr (TRAP) {
        const float cw = (pv_d + dd.x) * pv_hx;
        [&]<int... J>(std::integer_sequence<int, J...>) {
          (([&] {
             constexpr int j = J;
             const float a = __builtin_amdgcn_exp2f(dd.x * A2[j]);
             float g;
             if constexpr (TQ == 0) {
               g = __builtin_fmaf(cw, Bprev[j], h[j]);
             } else {
               constexpr int fp = bidx(TQ - 1, j);  // B_{t-1}[n0 + j]
               g = fmac_row_bcast<fp % 16>(h[j], rv[P][fp / 16], cw);
             }
             h[j] = a * g;
             if constexpr (FULL) {
               constexpr int fc = cidx(TQ, j);
               if constexpr (j == 0) yp = row_bcast<fc % 16>(rv[P][fc / 16]) * h[0];
               else yp = fmac_row_bcast<fc % 16>(yp, rv[P][fc / 16], h[j]);
             } else {
               asm volatile("" : "+v"(h[j]));
             }
           }()),
           ...);
        }(std::make_integer_sequence<int, NPL>{});
        pv_d = dd.x;
        pv_hx = dd.y;
        if constexpr (FULL) sY[P][w][TQ][lane] = yp;
        else block_delta += dd.x;
        return;
      }
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (([&] {
           constexpr int j = J;
           constexpr int fb = bidx(TQ, j);
           const float Bj = row_bcast<fb % 16>(rv[P][fb / 16]);
           const float a = __builtin_amdgcn_exp2f(dd.x * A2[j]);
           h[j] = __builtin_fmaf(a, h[j], dd.y * Bj);
           if constexpr (FULL) {
             constexpr int fc = cidx(TQ, j);
             if constexpr (j == 0) yp = row_bcast<fc % 16>(rv[P][fc / 16]) * h[0];
             else yp = fmac_row_bcast<fc % 16>(yp, rv[P][fc / 16], h[j]);
           } else {
             // Without the readout store nothing ties the update to its
             // token: the optimiser would sink a whole block of updates below
             // the next loads.  An empty asm with h as an in/out operand
             // keeps each update where it is written.
             asm volatile("" : "+v"(h[j]));
           }
         }()),
         ...);
      }(std::make_integer_sequence<int, NPL>{});
      if constexpr (FULL) sY[P][w][decltype(gc)::value * SUB + decltype(qc)::value][lane] = yp;
      else block_delta += dd.x;
    };

    // Double-buffered staged (delta, delta*u) of a group's tokens.
    float2 dd[2][SUB];
    auto fetch_dd = [&](auto parc, auto bufc, int g) {
      constexpr int P = decltype(parc)::value;
      constexpr int BUF = decltype(bufc)::value;
#pragma unroll
      for (int q = 0; q < SUB; ++q) dd[BUF][q] = sDU[P][g * SUB + q][lane];
    };

    // Group g of the block with parity P from buffer BUF: the next group's
    // staged values are fetched into the other buffer while this one computes.
    // (The only waits in the scan are on these LDS reads, which complete in
    // order, so the compiler's own wait counts and schedule are left free.)
    auto group = [&](auto parc, auto bufc, auto gc, float& block_delta) {
      constexpr int BUF = decltype(bufc)::value;
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 1 < NG) fetch_dd(parc, IC<1 - BUF>{}, g + 1);
      [&]<int... Q>(std::integer_sequence<int, Q...>) {
        (update(parc, gc, IC<Q>{}, dd[BUF][Q], block_delta), ...);
      }(std::make_integer_sequence<int, SUB>{});
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
      if constexpr (CKPT) {
        // the state entering block k (the padding blocks at the end have room too); under the
        // trapezoidal rule the registers hold h minus the previous token's delta (u/2) B (zero at a
        // pass's start), which the checkpoint adds back
#pragma unroll
        for (int j = 0; j < NPL; ++j)
          ckpt_row[static_cast<int64_t>(k) * 64 * NPAD + j] = TRAP ? __builtin_fmaf(pv_d * pv_hx, Bprev[j], h[j]) : h[j];
      }
      fetch_dd(parc, IC<0>{}, 0);
      if (k > k_begin) epilogue(IC<1 - P>{}, IC<Sm1>{}, k - 1);
      prologue(IC<1 - P>{}, IC<Sp1>{}, k + 1);
      issue_loads(IC<Sm1>{}, k + kPD + 1);
      load_records(IC<1 - P>{}, k + 1);
      float block_delta = 0.0f;
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((group(parc, IC<I % 2>{}, IC<I>{}, block_delta)), ...);
      }(std::make_integer_sequence<int, NG>{});
      if constexpr (TRAP) {
        // B of the block's last token, for the next block's first update
        [&]<int... J>(std::integer_sequence<int, J...>) {
          ((Bprev[J] = row_bcast<bidx(TB - 1, J) % 16>(rv[P][bidx(TB - 1, J) / 16])), ...);
        }(std::make_integer_sequence<int, NPL>{});
      }
      delta_total += block_delta;
      __syncthreads();
    };

    // fill the ring with blocks k_begin .. k_begin+kPD, stage block k_begin
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (issue_loads(IC<I>{}, k_begin + I), ...);
    }(std::make_integer_sequence<int, kPD + 1>{});
    load_records(IC<0>{}, k_begin);
    prologue(IC<0>{}, IC<0>{}, k_begin);
    __syncthreads();
    for (int k = k_begin; k < k_end; k += kRing) {
      const bool poll = stop_flag != nullptr && k + kRing >= k_stop;
      unsigned seen = 0u;
      if (poll && tid == 0) seen = __hip_atomic_load(stop_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (iteration(IC<I>{}, k + I), ...);
      }(std::make_integer_sequence<int, kRing>{});
      if (poll) {
        // Thread 0 hands the flag to every wavefront through that wavefront's
        // own word of the parity-0 partial readouts: the buffer is free at a
        // trip boundary (its last reader, the epilogue in the trip's last
        // block, is behind the barrier), and wavefront w next writes its word
        // in the following block's scan, after reading it.  Launches without
        // a readout never write that buffer otherwise.
        auto word = [&](int ww) -> float& {
          if constexpr (HAS_FULL) return sY[0][ww][TB - 1][63];
          else return sY[0][0][ww][63];
        };
        if (tid == 0) {
#pragma unroll
          for (int ww = 0; ww < G; ++ww) word(ww) = __builtin_bit_cast(float, seen);
        }
        __syncthreads();
        if (__builtin_bit_cast(unsigned, word(w)) != 0u) {
          k_end = k + kRing;
          stopped = true;
          break;
        }
      }
    }
    epilogue(IC<1>{}, IC<kRing - 1>{}, k_end - 1);  // k_end is a multiple of kRing (even)
    __syncthreads();  // the staging buffers are free for whatever runs next
    if (TRAP && !stopped) {
      // back from s to h: h = s + delta (u/2) B of the last token scanned (zero
      // after a padding token, whose step already made the same correction)
      const float e = pv_d * pv_hx;
#pragma unroll
      for (int j = 0; j < NPL; ++j) h[j] = __builtin_fmaf(e, Bprev[j], h[j]);
    }
    return delta_total;
  };

  // h_{-1} of the recurrence row `row` (batch row or packed sequence), when given
  auto init_state = [&](int64_t row) {
    if (p.h0 && dvalid) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (n0 + j < N) h[j] = p.h0[(row * dim + d) * N + n0 + j];
    }
  };
  auto write_final_state = [&](int64_t row) {
    if (dvalid && p.final_state) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (n0 + j < N) p.final_state[(row * dim + d) * N + n0 + j] = h[j];
    }
  };

  if constexpr (CHAINED) {
    constexpr bool FULLC = MODE == kModeChained;  // the chained checkpoint pass has no readout
    // One workgroup per CU.  Ticket j (the order workgroups start) owns
    // whole tile j and, for j < n_split * Ks, chunk c = j / n_split of
    // left-over tile n_long + j % n_split.  Chunk 0 runs first; chunk c > 0
    // is spliced in after about c chunk-lengths of the whole tile, by when the
    // workgroup running chunk c-1 (an earlier ticket) has handed on its final
    // state.  The whole tile's state waits in registers meanwhile.
    unsigned* sTicket = reinterpret_cast<unsigned*>(&sDU[0][0][0]);  // the staging buffer is not yet in use
    if (tid == 0) *sTicket = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int j = static_cast<int>(__builtin_amdgcn_readfirstlane(*sTicket));
    __syncthreads();  // every wavefront has read it before the buffer is written
    set_tile(j, 0, L);
    init_state(b);
    int nb_whole = stretch_blocks();
    const bool has_chunk = j < p.n_split * p.Ks;
    if (!has_chunk) {
      run_pass(IC<FULLC>{}, 0, nb_whole);
      write_final_state(b);
      return;
    }
    const int c = j / p.n_split, st = j % p.n_split;
    const int64_t cb = static_cast<int64_t>(c) * p.chunk_len;
    const int64_t ce = (cb + p.chunk_len < L) ? cb + p.chunk_len : L;
    const int nb_chunk = static_cast<int>((ce - cb + TRIP - 1) / TRIP) * kRing;
    // Splice point: not before c chunks' worth of blocks, and only once chunk
    // c-1 has handed on its state (chunk 0 goes first).
    int m = c * nb_chunk;
    if (m > nb_whole) m = nb_whole;
    const unsigned* my_flag = p.wait_override ? p.wait_override : p.flags + static_cast<int64_t>(st) * p.Ks + c;
    if (c > 0) {
      m = nb_whole;
      run_pass(IC<FULLC>{}, 0, m, my_flag, c * nb_chunk);
    }
    float hw[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      hw[q] = h[q];
      h[q] = 0.0f;
    }
    set_tile(p.n_long + st, cb, ce);
    if (c == 0) init_state(b);
    const int64_t crow = (static_cast<int64_t>(st) * p.Ks + c) * 64 + lane;  // carry row [n_split][Ks][64]
    // The carries and flags are read and written only with device-coherent
    // (agent-scope) loads and stores, which bypass the per-XCD L2s; waiting
    // for the carry stores to complete before the flag store orders them.
    // (Release/acquire fences would instead write back or invalidate the
    // whole L2, slowing every workgroup on the XCD.)
    if (c > 0) {
      // the staging buffer is free between passes: its first word carries the outcome of the wait
      if (tid == 0) {
        const bool ok = poll_ready(my_flag, p.spin_limit);
        if (!ok) __hip_atomic_fetch_or(p.status, kStatusHandoffTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *sTicket = ok ? 1u : 0u;
      }
      __syncthreads();
      const bool lost = *sTicket == 0u;  // this wait ran out (not another's)
      __syncthreads();  // read by every wavefront before the pass stages into the buffer
      if (dvalid) {
#pragma unroll
        for (int q = 0; q < NPL; ++q)
          h[q] = lost ? __builtin_nanf("")
                      : __hip_atomic_load(p.carry + crow * NPAD + n0 + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    int nbc = nb_chunk;
    run_pass(IC<FULLC>{}, 0, nbc);
    if (c + 1 < p.Ks) {
      if (dvalid) {
#pragma unroll
        for (int q = 0; q < NPL; ++q)
          __hip_atomic_store(p.carry + (crow + 64) * NPAD + n0 + q, h[q], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this thread's carry stores have completed
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(p.flags + static_cast<int64_t>(st) * p.Ks + c + 1, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      write_final_state(b);
    }
    set_tile(j, 0, L);
#pragma unroll
    for (int q = 0; q < NPL; ++q) h[q] = hw[q];
    run_pass(IC<FULLC>{}, m, nb_whole, nullptr, 0, true);  // resumes h as the first part left it
    write_final_state(b);
  } else {
    // ---- which tile and which part of the sequence this workgroup scans
    const int unit = blockIdx.x;
    int tile, c, st;
    bool split;
    constexpr bool PACKABLE = MODE == kModeFull || MODE == kModeCkpt;  // modes that run packed sequences
    if ((MODE == kModeCkpt && p.cu == nullptr) || (MODE == kModeFull && unit < p.n_long)) {
      tile = unit;
      c = 0;
      st = 0;
      split = false;
    } else {
      const int per = MODE == kModeFull ? p.Ks : p.Ks - 1;
      const int jj = MODE == kModeFull ? unit - p.n_long : unit;
      if (PACKABLE && p.cu != nullptr) {  // packed: every tile column of a sequence together
        st = jj % p.n_split;
        c = p.order ? p.order[jj / p.n_split] : jj / p.n_split;
      } else {
        st = jj / per;
        c = jj % per;
      }
      tile = p.n_long + st;
      split = true;
    }
    int64_t tb = split ? static_cast<int64_t>(c) * p.chunk_len : 0;
    int64_t te = split ? ((tb + p.chunk_len < L) ? tb + p.chunk_len : L) : L;
    const bool packed = PACKABLE && split && p.cu != nullptr;
    if (packed) {  // sequence c of batch row 0, offsets clamped into [0, L]
      tb = p.cu[c];
      tb = tb < 0 ? 0 : (tb > L ? L : tb);
      te = p.cu[c + 1];
      te = te < tb ? tb : (te > L ? L : te);
    }
    set_tile(tile, tb, te);
    if (packed) row_start = true;  // a packed sequence has no input before its first token
    if (CKPT && packed) ckpt_row += static_cast<int64_t>(kPackedCkptSlack) * c * 64 * NPAD;
    const int64_t pair_row = (static_cast<int64_t>(st) * p.Ks + c) * 64 + lane;   // row of [n_split][Ks][64]
    if constexpr (MODE == kModeCkpt) {
      init_state(packed ? c : b);
      int nb = stretch_blocks();
      run_pass(IC<false>{}, 0, nb);
    } else if constexpr (MODE == kModeAgg) {
      // chunk pair from a zero state: S = h, P = exp(A * sum of deltas)
      int nb = stretch_blocks();
      const float dt = run_pass(IC<false>{}, 0, nb);
      if (!dvalid) return;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const int64_t idx = pair_row * NPAD + n0 + q;
        p.aggS[idx] = h[q];
        p.aggP[idx] = __builtin_amdgcn_exp2f(A2[q] * dt);
      }
    } else {
      if (packed) {
        init_state(c);
      } else if (!split || c == 0) {
        init_state(b);
      } else if (dvalid) {
#pragma unroll
        for (int q = 0; q < NPL; ++q) h[q] = p.carry[pair_row * NPAD + n0 + q];
      }
      int nb = stretch_blocks();
      run_pass(IC<true>{}, 0, nb);
      if (packed) write_final_state(c);
      else if (!split || c == p.Ks - 1) write_final_state(b);
    }
  }
}

}  // namespace ssm
