// lane_kernels.hpp -- the selective scan with one channel per lane.
//
// Each lane owns one channel d of one batch row and all NS of its states, in
// registers; a wavefront covers 64 consecutive channels (a tile) over one
// chunk of the sequence.  B_t and C_t are the same for the whole wavefront:
// they arrive as one register each holding B_t[n] (C_t[n]) in lane n of every
// 16-lane row, and every update reads them with a DPP row broadcast.  Nothing
// is shared between wavefronts (no LDS, no barrier), and the readout
// y_t = sum_n C_t[n] h_t[n] is summed inside the lane.
//
// A tile is one wavefront, so the sequence is cut into many chunks to fill the
// GPU, and the chunks are stitched through their fade-and-add pairs ("Mamba is
// attention all you really need, part 2", "The relay"):
//   pair pass (FULL = false): chunks 0..K-2 of every tile from a zero state:
//             S = the state the chunk reaches, P = its total fade;
//   carry_kernel: the state entering every chunk;
//   full pass (FULL = true): every chunk from its carried-in state, giving y
//             and, for the last chunk, the final state.
//
// Fades.  With a general A, a_n = exp(delta A[d,n]): one exp per state update.
// With the structured A[d,n] = (n+1) a0[d], a_n = q^(n+1) for q = exp(delta
// a0): one exp per (token, channel), the powers by repeated multiplication.
// The structured pair pass walks its chunk backwards and sums
//   S_n = sum_s (prod_{r>s} q_r)^(n+1) delta_s u_s B_s[n],
// with Q_s = prod_{r>s} q_r = exp(a0 * sum_{r>s} delta_r): one exp per
// (token, channel), and per state one multiply (the next power of Q times
// delta u) and one fma.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "common.hpp"

namespace ssm {

struct LaneParams {
  const void* u;
  const void* delta;
  const float* A;      // general: A [dim][N]; structured: a0 [dim], A[d,n] = (n+1) a0[d]
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  // B and C: packed fp32 records [batch][Lp][32] (B_t in floats 0..15, C_t in 16..31, zero past N), or
  // null for fp32 storage, whose rows [batch][L][N] are read directly.
  const float* bc;
  int64_t bc_rows;     // records in bc (batch * Lp plus the zero padding past the last row)
  const void* Braw;
  const void* Craw;
  void* y;
  float* final_state;  // nullable
  const float* h0;     // nullable: [batch][dim][N], the state before token 0
  // Chunk pairs and carried-in states, [n_tiles][K][64][NS].
  float* aggP;
  float* aggS;
  float* carry;
  int64_t batch, L, Lp, dim, N;
  int64_t chunk_len;   // tokens per chunk (the last may be shorter)
  int ntd;             // 64-channel tiles per batch row
  int n_tiles;         // batch * ntd
  int K;               // chunks per tile
  int softplus;
};

constexpr int kLaneTG = 4;     // tokens per software-pipelined group of loads
constexpr int kLaneWaves = 4;  // independent wavefronts per workgroup

// Raw loads of one token: u, delta_raw, z (bf16 in the low half, or fp32 bits), and the B, C registers.
struct LaneTok {
  uint32_t u, d, z;
  float B, C;
};

template <class IO> __device__ __forceinline__ uint32_t lane_load(rsrc_t r, unsigned off, int soff) {
  if constexpr (__is_same(IO, F32))
    return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), soff, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), soff, 0);
}
template <class IO> __device__ __forceinline__ float lane_value(uint32_t raw) {
  if constexpr (__is_same(IO, F32)) return __uint_as_float(raw);
  else return __uint_as_float(raw << 16);
}
template <class IO> __device__ __forceinline__ void lane_store(rsrc_t r, unsigned off, int soff, float v) {
  if constexpr (__is_same(IO, F32))
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(off), soff, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b16(to_bf16(v), r, static_cast<int>(off), soff, 0);
}

template <class IO, int NS, bool STRUCT, bool FULL, bool GATE>
__global__ void __launch_bounds__(64 * kLaneWaves) lane_scan_kernel(LaneParams p) {
  static_assert(FULL || !GATE, "the gate belongs to the full pass");
  static_assert(NS == 4 || NS == 8 || NS == 16, "states per lane");
  constexpr int ES = __is_same(IO, F32) ? 4 : 2;
  constexpr int TG = kLaneTG;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kLaneWaves + wv;
  const int64_t n_units = static_cast<int64_t>(p.n_tiles) * (FULL ? p.K : p.K - 1);
  if (unit >= n_units) return;  // a whole wavefront
  const int c = static_cast<int>(unit / p.n_tiles);
  const int tile = static_cast<int>(unit % p.n_tiles);
  const int64_t L = p.L, dim = p.dim, N = p.N;
  const int64_t b = tile / p.ntd;
  const int64_t d0 = static_cast<int64_t>(tile % p.ntd) * 64;
  const int64_t d = d0 + lane;
  const bool dvalid = d < dim;
  const int64_t t0 = static_cast<int64_t>(c) * p.chunk_len;
  const int64_t t1 = (t0 + p.chunk_len < L) ? t0 + p.chunk_len : L;
  const int nt = static_cast<int>(t1 - t0);

  // Token rows of u, delta_raw, z, y through buffer resources covering (b, t0, d0) to the end of the
  // chunk's last row: tokens past the chunk read zero and are not written.  A group of TG tokens is
  // addressed by the (scalar) offset of its first row plus a lane's fixed offset of each token in it.  A
  // channel past dim gets offsets at or above 2^31, past the range (the host keeps a chunk and its
  // padding below 2^31 bytes).
  const unsigned row_bytes = static_cast<unsigned>(dim * ES);
  const int64_t base = ((b * L + t0) * dim + d0) * ES;
  const int64_t bytes = static_cast<int64_t>(nt) * row_bytes - d0 * ES;
  const rsrc_t rs_u = make_rsrc(static_cast<const char*>(p.u) + base, bytes);
  const rsrc_t rs_d = make_rsrc(static_cast<const char*>(p.delta) + base, bytes);
  constexpr bool has_z = GATE;  // the host launches GATE exactly when z is given
  const rsrc_t rs_z = make_rsrc(has_z ? static_cast<const char*>(p.z) + base : nullptr, has_z ? bytes : 0);
  const rsrc_t rs_y = make_rsrc(FULL ? static_cast<char*>(p.y) + base : nullptr, FULL ? bytes : 0);
  const unsigned lo = dvalid ? static_cast<unsigned>(lane * ES) : 0x80000000u;
  // B and C: lane l reads state l % 16 of each token (zero past N)
  rsrc_t rs_B, rs_C;
  unsigned b_lo, c_lo, bc_stride;
  int64_t bc_bytes;
  if (p.bc) {
    const float* rec = p.bc + (b * p.Lp + t0) * 32;
    bc_bytes = (p.bc_rows - b * p.Lp - t0) * 32 * static_cast<int64_t>(sizeof(float));
    rs_B = make_rsrc(rec, bc_bytes);
    rs_C = rs_B;
    b_lo = static_cast<unsigned>((lane & 15) * 4);
    c_lo = b_lo + 64u;
    bc_stride = 128u;
  } else {
    const int64_t rb = (b * L + t0) * N * static_cast<int64_t>(sizeof(float));
    bc_bytes = (L - t0) * N * static_cast<int64_t>(sizeof(float));
    if (bc_bytes > 0x7fffffffLL) bc_bytes = 0x7fffffffLL;
    rs_B = make_rsrc(static_cast<const char*>(p.Braw) + rb, bc_bytes);
    rs_C = make_rsrc(static_cast<const char*>(p.Craw) + rb, bc_bytes);
    b_lo = (lane & 15) < N ? static_cast<unsigned>((lane & 15) * 4) : 0x80000000u;
    c_lo = b_lo;
    bc_stride = static_cast<unsigned>(N * 4);
  }
  // Token j of a group sits at row jr = j (forward) or TG-1-j (backward) from the group's first row.
  constexpr bool BACKWARD = STRUCT && !FULL;
  unsigned tok_off[TG], rec_off[TG];
#pragma unroll
  for (int j = 0; j < TG; ++j) {
    const unsigned jr = BACKWARD ? TG - 1 - j : j;
    tok_off[j] = lo + jr * static_cast<unsigned>(row_bytes);
    rec_off[j] = b_lo + jr * bc_stride;
  }

  // per-channel constants
  float A2[STRUCT ? 1 : NS];
  if constexpr (STRUCT) {
    A2[0] = dvalid ? p.A[d] * kLog2e : 0.0f;
  } else {
#pragma unroll
    for (int n = 0; n < NS; ++n) A2[n] = (dvalid && n < N) ? p.A[d * N + n] * kLog2e : 0.0f;
  }
  const float biasv = (dvalid && p.bias) ? p.bias[d] : 0.0f;
  const float Dv = (dvalid && p.D) ? p.D[d] : 0.0f;
  const float sp_k = p.softplus != 0 ? 1.0f : 0.0f;
  const float sp_lo = p.softplus != 0 ? 0.0f : -__builtin_inff();

  // h: the state (full pass) or the chunk's S (pair pass)
  float h[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) h[n] = 0.0f;
  const int64_t prow = ((static_cast<int64_t>(tile) * p.K + c) * 64 + lane) * NS;  // row of [n_tiles][K][64][NS]
  if constexpr (FULL) {
    if (c == 0) {
      if (p.h0 && dvalid) {
#pragma unroll
        for (int n = 0; n < NS; ++n)
          if (n < N) h[n] = p.h0[(b * dim + d) * N + n];
      }
    } else {
#pragma unroll
      for (int v = 0; v < NS / 4; ++v) {
        const float4 x = reinterpret_cast<const float4*>(p.carry + prow)[v];
        h[4 * v] = x.x;
        h[4 * v + 1] = x.y;
        h[4 * v + 2] = x.z;
        h[4 * v + 3] = x.w;
      }
    }
  }

  // Group g of the walk: tokens g*TG .. g*TG+TG-1 of the chunk (forward), or tokens nt-1-g*TG down to
  // nt-TG-g*TG (the structured pair pass walks backwards; its chunks, all but the sequence's last, are
  // whole groups).  The scalar offsets of the group's first row in the token rows and in the B/C rows.  A
  // group wholly past the chunk is only prefetched, never computed: its token offset is the range's size
  // (it reads zero), its record offset the records' size or 2^31 - 1, whichever is less (past 2^31 - 1
  // bytes of records it may read records of later tokens).
  auto first_row = [&](int g) -> int {
    if constexpr (BACKWARD) return g * TG < nt ? nt - TG - g * TG : -1;
    else return g * TG < nt ? g * TG : -1;
  };
  auto tok_soff = [&](int g) -> int {
    const int r0 = first_row(g);
    return r0 < 0 ? static_cast<int>(bytes) : r0 * static_cast<int>(row_bytes);
  };
  const int bc_past = static_cast<int>(bc_bytes < 0x7fffffffLL ? bc_bytes : 0x7fffffffLL);
  auto rec_soff = [&](int g) -> int {
    const int r0 = first_row(g);
    return r0 < 0 ? bc_past : r0 * static_cast<int>(bc_stride);
  };
  auto issue = [&](LaneTok (&r)[TG], int g) {
    const int so = tok_soff(g), sr = rec_soff(g);
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      r[j].u = lane_load<IO>(rs_u, tok_off[j], so);
      r[j].d = lane_load<IO>(rs_d, tok_off[j], so);
      if constexpr (has_z) r[j].z = lane_load<IO>(rs_z, tok_off[j], so);
      r[j].B = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_B, static_cast<int>(rec_off[j]), sr, 0));
      if constexpr (FULL)
        r[j].C = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rs_C, static_cast<int>(rec_off[j] + (c_lo - b_lo)), sr, 0));
    }
  };

  float sfx = 0.0f;  // pair passes: the sum of the steps walked so far
  // A group's per-(token, channel) values first (independent of the state, so their exps and logs overlap
  // the updates of the tokens before them), then its updates in order.  The powers of q (and Q) run as two
  // chains of alternate states and the readout as two partial sums, so no long dependency chain stalls a
  // wavefront that has a SIMD to itself.
  // MASK: the group may hold tokens past the chunk, which take the identity step (1, 0).
  auto compute = [&](LaneTok (&r)[TG], int g, auto maskc) {
    constexpr bool MASK = decltype(maskc)::value != 0;
    float dl[TG], du[TG], q[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      float x = step_of(lane_value<IO>(r[j].d) + biasv, sp_k, sp_lo);
      dl[j] = (!MASK || g * TG + j < nt) ? x : 0.0f;
      du[j] = dl[j] * lane_value<IO>(r[j].u);
      if constexpr (STRUCT && FULL) q[j] = __builtin_amdgcn_exp2f(dl[j] * A2[0]);
    }
    const int so = FULL ? tok_soff(g) : 0;
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      if constexpr (FULL) {
        float y0 = 0.0f, y1 = 0.0f;
        if constexpr (STRUCT) {
          const float q2 = q[j] * q[j];
          float a0 = q[j], a1 = q2;  // fades of states 2m and 2m+1: q^(2m+1), q^(2m+2)
          [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
               constexpr int n = I;
               const float a = (n & 1) ? a1 : a0;
               h[n] = __builtin_fmaf(a, h[n], row_bcast<n>(r[j].B) * du[j]);
               if constexpr (n == 0) y0 = row_bcast<0>(r[j].C) * h[0];
               else if constexpr (n == 1) y1 = row_bcast<1>(r[j].C) * h[1];
               else if constexpr (n & 1) y1 = fmac_row_bcast<n>(y1, r[j].C, h[n]);
               else y0 = fmac_row_bcast<n>(y0, r[j].C, h[n]);
               if constexpr (n + 2 < NS) {
                 if constexpr (n & 1) a1 *= q2;
                 else a0 *= q2;
               }
             }()),
             ...);
          }(std::make_integer_sequence<int, NS>{});
        } else {
          [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
               constexpr int n = I;
               const float a = __builtin_amdgcn_exp2f(dl[j] * A2[n]);
               h[n] = __builtin_fmaf(a, h[n], row_bcast<n>(r[j].B) * du[j]);
               if constexpr (n == 0) y0 = row_bcast<0>(r[j].C) * h[0];
               else if constexpr (n == 1) y1 = row_bcast<1>(r[j].C) * h[1];
               else if constexpr (n & 1) y1 = fmac_row_bcast<n>(y1, r[j].C, h[n]);
               else y0 = fmac_row_bcast<n>(y0, r[j].C, h[n]);
             }()),
             ...);
          }(std::make_integer_sequence<int, NS>{});
        }
        float out = __builtin_fmaf(Dv, lane_value<IO>(r[j].u), y0 + y1);
        if constexpr (has_z) out *= silu_f(lane_value<IO>(r[j].z));
        lane_store<IO>(rs_y, tok_off[j], so, out);
      } else if constexpr (STRUCT) {
        // backwards: Q = prod over the tokens after this one of q
        const float Q = __builtin_amdgcn_exp2f(A2[0] * sfx);
        sfx += dl[j];
        const float Q2 = Q * Q;
        float v0 = du[j] * Q, v1 = v0 * Q;  // du Q^(2m+1), du Q^(2m+2)
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (([&] {
             constexpr int n = I;
             if constexpr (n & 1) {
               h[n] = fmac_row_bcast<n>(h[n], r[j].B, v1);
               if constexpr (n + 2 < NS) v1 *= Q2;
             } else {
               h[n] = fmac_row_bcast<n>(h[n], r[j].B, v0);
               if constexpr (n + 2 < NS) v0 *= Q2;
             }
           }()),
           ...);
        }(std::make_integer_sequence<int, NS>{});
      } else {
        sfx += dl[j];
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (([&] {
             constexpr int n = I;
             const float a = __builtin_amdgcn_exp2f(dl[j] * A2[n]);
             h[n] = __builtin_fmaf(a, h[n], row_bcast<n>(r[j].B) * du[j]);
           }()),
           ...);
        }(std::make_integer_sequence<int, NS>{});
      }
    }
  };

  // groups of TG tokens, two register sets: group g+1 loads while group g computes; pairs of groups
  // wholly inside the chunk first, then (only in a chunk that ends ragged, the sequence's last) a masked
  // pair holding its end
  LaneTok r0[TG], r1[TG];
  const int ng = (nt + TG - 1) / TG;
  const int ngf = nt / (2 * TG) * 2;
  issue(r0, 0);
  int g = 0;
  // The scheduling barriers keep each group's loads where they are written, a whole group ahead of
  // their use: their offsets need no vector work, and left free the scheduler sinks them next to it.
  for (; g < ngf; g += 2) {
    issue(r1, g + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(r0, g, IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
    issue(r0, g + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(r1, g + 1, IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
  }
  if (g < ng) {
    const bool two = g + 1 < ng;
    if (two) issue(r1, g + 1);
    compute(r0, g, IC<1>{});
    if (two) compute(r1, g + 1, IC<1>{});
  }

  if constexpr (FULL) {
    if (c == p.K - 1 && p.final_state && dvalid) {
#pragma unroll
      for (int n = 0; n < NS; ++n)
        if (n < N) p.final_state[(b * dim + d) * N + n] = h[n];
    }
  } else {
    float P[NS];
    if constexpr (STRUCT) {
      const float e = A2[0] * sfx;
#pragma unroll
      for (int n = 0; n < NS; ++n) P[n] = __builtin_amdgcn_exp2f(static_cast<float>(n + 1) * e);
    } else {
#pragma unroll
      for (int n = 0; n < NS; ++n) P[n] = __builtin_amdgcn_exp2f(A2[n] * sfx);
    }
#pragma unroll
    for (int v = 0; v < NS / 4; ++v) {
      reinterpret_cast<float4*>(p.aggS + prow)[v] = make_float4(h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]);
      reinterpret_cast<float4*>(p.aggP + prow)[v] = make_float4(P[4 * v], P[4 * v + 1], P[4 * v + 2], P[4 * v + 3]);
    }
  }
}

// Launch of the pair pass (full = false) or the full pass over a grid of
// ceil(units / kLaneWaves) workgroups; ns: states per lane (4, 8 or 16);
// structured: A holds a0 [dim]; the gate is applied when p.z is set.
// Instantiated in scan_lane.hip.
template <class IO>
hipError_t launch_lane(int ns, bool structured, bool full, const LaneParams& p, hipStream_t s);
extern template hipError_t launch_lane<F32>(int, bool, bool, const LaneParams&, hipStream_t);
extern template hipError_t launch_lane<BF16>(int, bool, bool, const LaneParams&, hipStream_t);

}  // namespace ssm
