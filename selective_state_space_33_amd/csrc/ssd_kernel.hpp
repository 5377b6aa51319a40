// ssd_kernel.hpp -- the Mamba-2 state-space-duality (SSD) layer on MFMA.
//
// Mamba-2 gives every head one scalar state matrix A (times the identity), so
// the sequence map of a head is multiplication by a causal 1-semiseparable
// matrix and can be computed blockwise with matrix products ("State Space
// Models and the Post-Transformer Era", "Mamba-2 and Structured State Space
// Duality"; "The State That Must Remember Everything", Part 4).  Per batch row
// and head (headdim P = 64 channels sharing delta_t and A, with B_t, C_t of
// dstate N shared by all heads) the state H (N x P) runs
//     H_t = exp(delta_t A) H_{t-1} + delta_t B_t x_t^T,   y_t = H_t^T C_t + D x_t,
// then y is gated by SiLU(z).  Over a chunk of Q tokens with
// cs_t = A (delta_0 + ... + delta_t) (chunk-local, inclusive) this is
//     y_t   = exp(cs_t) H_prev^T C_t                                  (inter)
//           + sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) delta_s x_s        (intra)
//     H_end = exp(cs_end) H_prev + sum_s exp(cs_end - cs_s) delta_s B_s x_s^T.
//
// One workgroup (16 wavefronts, 8 for dstate 32) per (batch row, head) walks the chunks in
// order; the head's state stays in MFMA accumulators (fp32), so no chunk
// state goes to HBM and x, z, y, B, C are each read or written once.  Per
// chunk (v_mfma_f32_16x16x32_bf16, bf16 operands, fp32 accumulation):
//   G^T = B C^T              (Q x Q, K = N) -> M[t][s] = G[t][s] exp(cs_t - cs_s) delta_s on s <= t
//   Y   = exp(cs_t) C H + M x  (Q x P; K = N, then K = Q)  -> + D x, times SiLU(z), y
//   H   = exp(cs_end) H + W^T x   (N x P, K = Q),  W[s][n] = exp(cs_end - cs_s) delta_s B[s][n]
// Every operand sits in LDS with its K index contiguous, so a fragment is one
// 16-byte read: C and B by token row, M by output row, x, W and H transposed
// (x^T [p][s], W^T [n][s], H^T [p][n]).  The orientations are chosen so that
// every write is an 8-byte run: the accumulators of G^T and H hold four
// consecutive K-side indices per lane, and B and x are loaded four token rows
// at a time so that their transposes are written four tokens per store.
//
// Precision.  C, B and x arrive as bf16 and are exact operands.  M, W and the
// state are fp32 values; rounded to bf16 once, the sums they enter lose about
// 2^-9 of their largest terms, which against the fp64 oracle puts y near 2e-2
// of its scale.  Each of the three is therefore carried as a pair hi + lo of
// bf16 (hi = bf16(v), lo = bf16(v - hi)) and enters its product as two
// MFMAs, which keeps y at the rounding of its own bf16 store (~4e-3) and the
// state near 2e-5.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ssm {

struct SsdParams {
  const void* x;       // [batch][L][H][P] bf16
  const void* delta;   // [batch][L][H] bf16 (raw)
  const float* A;      // [H]
  const void* B;       // [batch][L][N] bf16
  const void* C;       // [batch][L][N] bf16
  const float* D;      // [H] (nullable)
  const void* z;       // [batch][L][H][P] bf16 (nullable)
  const float* bias;   // [H] (nullable)
  void* y;             // [batch][L][H][P] bf16
  float* final_state;  // [batch][H][P][N] (nullable)
  const float* h0;     // [batch][H][P][N]: the state before token 0 (nullable: zero)
  int64_t batch, L, H;
  int softplus;
  // Chained launches (n_split > 0): units (batch row, head) 0 .. n_long-1
  // whole, n_long .. n_long+n_split-1 cut into Ks segments of seg_chunks
  // chunks, states handed on through carry [n_split][Ks][P][N] and flags
  // [n_split][Ks], with a workgroup ticket and a status word (all zeroed
  // before the launch).
  int n_long, n_split, Ks;
  int64_t seg_chunks;
  float* carry;
  unsigned* flags;
  unsigned* ticket;
  unsigned* status;
};

// A chained segment waits for the state handed on to it for at most this
// many polls (each after a short sleep); past that it records an error bit in
// the status word and goes on from a NaN state, so the kernel always ends and
// the outputs that depend on the lost hand-off show the failure.
constexpr unsigned kSsdSpinLimit = 1u << 18;
constexpr int kSsdWaitVm0 = 0x0F70;  // vmcnt(0), other counters at their maxima (gfx9 s_waitcnt)

// Zeroes the flags, ticket and status of a chained launch.
__global__ void __launch_bounds__(256) ssd_zero_words_kernel(unsigned* words, int n) {
  for (int e = threadIdx.x; e < n; e += 256) words[e] = 0u;
}

constexpr int kSsdQ = 64;         // tokens per chunk
constexpr int kSsdP = 64;         // channels per head
// Wavefronts per workgroup: 16 (four per SIMD) where the state has at least
// 64 tiles of work to share, else 8.
constexpr int ssd_waves(int N) { return N >= 64 ? 16 : 8; }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned short bf16_bits_of(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_value(unsigned short b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
__device__ __forceinline__ float bf16_lo_of(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi_of(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// hi and lo bf16 of four fp32 values, packed as two 8-byte runs.
__device__ __forceinline__ void split4(const float* v, u32x2_t& hi, u32x2_t& lo) {
  unsigned short hb[4], lb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hb[j] = bf16_bits_of(v[j]);
    lb[j] = bf16_bits_of(v[j] - bf16_value(hb[j]));
  }
  hi = u32x2_t{hb[0] | (static_cast<uint32_t>(hb[1]) << 16), hb[2] | (static_cast<uint32_t>(hb[3]) << 16)};
  lo = u32x2_t{lb[0] | (static_cast<uint32_t>(lb[1]) << 16), lb[2] | (static_cast<uint32_t>(lb[3]) << 16)};
}

template <int N>
__global__ void __launch_bounds__(64 * ssd_waves(N)) ssd_kernel(SsdParams p) {
  constexpr int Q = kSsdQ, P = kSsdP, NW = ssd_waves(N), NTH = 64 * NW;
  static_assert(N == 32 || N == 64 || N == 128, "dstate: 32, 64 or 128");
  constexpr int SN = N + 8;  // padded rows (elements) of the [.][N] arrays: 16-byte aligned, banks staggered
  constexpr int SQ = Q + 8;  // padded rows of the [.][Q] arrays
  constexpr int NT = N / 16;  // 16-wide state tiles
  constexpr int HT = NT * 4 / NW;  // state tiles per wavefront (NT x 4 tiles over NW wavefronts)
  constexpr int YT = 16 / NW;      // Y tiles per wavefront (4 x 4 over NW wavefronts)
  constexpr int XI = (Q / 4) * (P / 2);  // x items (4 tokens x 2 channels), one per thread up to XI
  constexpr int C_PIECES = Q * N / 8;         // 16-byte pieces of a chunk's C
  constexpr int C_PER = (C_PIECES + NTH - 1) / NTH;
  constexpr int B_ITEMS = (Q / 4) * (N / 2);  // (4 tokens) x (2 states) items of a chunk's B
  constexpr int B_PER = (B_ITEMS + NTH - 1) / NTH;
  static_assert(XI <= NTH && HT >= 1 && YT >= 1, "work split");
  constexpr float kLog2eF = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) unsigned short sC[Q * SN];   // C [t][n]
  __shared__ __attribute__((aligned(16))) unsigned short sB[Q * SN];   // B [s][n]
  __shared__ __attribute__((aligned(16))) unsigned short sWh[N * SQ];  // W^T [n][s], hi
  __shared__ __attribute__((aligned(16))) unsigned short sWl[N * SQ];  // lo
  __shared__ __attribute__((aligned(16))) unsigned short sXT[P * SQ];  // x^T [p][s]
  __shared__ __attribute__((aligned(16))) unsigned short sZT[P * SQ];  // z^T [p][t]
  __shared__ __attribute__((aligned(16))) unsigned short sMh[Q * SQ];  // M [t][s], hi
  __shared__ __attribute__((aligned(16))) unsigned short sMl[Q * SQ];  // lo
  __shared__ __attribute__((aligned(16))) unsigned short sHh[P * SN];  // H^T [p][n], hi
  __shared__ __attribute__((aligned(16))) unsigned short sHl[P * SN];  // lo
  // per chunk parity: A * (cumulative step) within the chunk, and the step delta_t; wavefront 0
  // prepares the next chunk's while the others finish the current one
  __shared__ __attribute__((aligned(16))) float sCS[2][Q];
  __shared__ __attribute__((aligned(16))) float sDL[2][Q];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t H = p.H, L = p.L;
  // elements between token rows of x, z, y; the host keeps every token-row
  // byte offset (one chunk past L included) below 2^31, so offsets are 32-bit
  const int rowe = static_cast<int>(H * P);
  const int H32 = static_cast<int>(H);

  // ---- the unit (batch row b, head h) being worked on
  int64_t b = 0, h = 0;
  float Ah = 0.0f, Dh = 0.0f, biash = 0.0f;
  rsrc_t rs_x, rs_z, rs_y, rs_b, rs_c, rs_d;
  auto set_unit = [&](int64_t unit) {
    b = unit / H;
    h = unit % H;
    Ah = p.A[h];
    Dh = p.D ? p.D[h] : 0.0f;
    biash = p.bias ? p.bias[h] : 0.0f;
    // Buffer resources: token rows past L read as zero and are not written.
    const int64_t xbase = (b * L * H + h) * P;
    const int64_t xbytes = (L * H - h) * P * 2;
    rs_x = make_rsrc(static_cast<const unsigned short*>(p.x) + xbase, xbytes);
    rs_z = make_rsrc(p.z ? static_cast<const unsigned short*>(p.z) + xbase : nullptr, p.z ? xbytes : 0);
    rs_y = make_rsrc(static_cast<unsigned short*>(p.y) + xbase, xbytes);
    rs_b = make_rsrc(static_cast<const unsigned short*>(p.B) + b * L * N, L * N * 2);
    rs_c = make_rsrc(static_cast<const unsigned short*>(p.C) + b * L * N, L * N * 2);
    rs_d = make_rsrc(static_cast<const unsigned short*>(p.delta) + b * L * H + h, (L * H - h) * 2);
  };

  // Work of this wavefront.  Y tiles: token block ty, channel blocks py0 .. py0+YT-1.
  const int ty = w & 3, py0 = YT * (w >> 2);
  // State tiles: channel block ph, state blocks nb0 + (NW/4) i.
  const int ph = w & 3, nb0 = w >> 2;
  constexpr int NBS = NW / 4;

  // Chunk loads (registers), one chunk ahead: C in 16-byte pieces; B, x and z
  // four token rows at a time (4-byte pieces: two states / two channels); the
  // raw step.  x and z are staged transposed, so that the epilogue reads the
  // z of four consecutive tokens as one 8-byte piece.
  u32x4_t gc[C_PER];
  uint32_t gb[B_PER][4], gx[4], gzz[4];
  float graw = 0.0f;
  auto load_c = [&](int t0) {
#pragma unroll
    for (int i = 0; i < C_PER; ++i) {
      const int e = tid + NTH * i;
      const int row = e / (N / 8), col = (e % (N / 8)) * 8;
      if (e < C_PIECES)
        gc[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rs_c, ((t0 + row) * N + col) * 2, 0, 0));
    }
  };
  auto load_b = [&](int t0) {
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int e = tid + NTH * i;
      const int np = e % (N / 2), s0 = 4 * (e / (N / 2));
      if (e < B_ITEMS) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gb[i][r] = __builtin_amdgcn_raw_buffer_load_b32(rs_b, ((t0 + s0 + r) * N + 2 * np) * 2, 0, 0);
      }
    }
  };
  const int xpp = tid % (P / 2), xs0 = 4 * (tid / (P / 2));  // x item: channels 2xpp, 2xpp+1 of tokens xs0..xs0+3
  auto load_x = [&](int t0) {
    if (tid < XI) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        gx[r] = __builtin_amdgcn_raw_buffer_load_b32(rs_x, ((t0 + xs0 + r) * rowe + 2 * xpp) * 2, 0, 0);
      if (p.z) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gzz[r] = __builtin_amdgcn_raw_buffer_load_b32(rs_z, ((t0 + xs0 + r) * rowe + 2 * xpp) * 2, 0, 0);
      }
    }
    if (w == 0)
      graw = bf16_value(static_cast<unsigned short>(__builtin_amdgcn_raw_buffer_load_b16(
          rs_d, (t0 + lane) * H32 * 2, 0, 0)));
  };
  f32x4_t hacc[HT];
  // H^T as bf16 pairs for the Y products, from the accumulators: four
  // consecutive states of one channel per lane (this wavefront's tiles only)
  auto stage_state = [&]() {
#pragma unroll
    for (int i = 0; i < HT; ++i) {
      const float v[4] = {hacc[i][0], hacc[i][1], hacc[i][2], hacc[i][3]};
      u32x2_t hi, lo;
      split4(v, hi, lo);
      const int idx = (16 * ph + lr) * SN + 16 * (nb0 + NBS * i) + 4 * lq;
      *reinterpret_cast<u32x2_t*>(&sHh[idx]) = hi;
      *reinterpret_cast<u32x2_t*>(&sHl[idx]) = lo;
    }
  };
  // state element (channel, state) of this lane's tile i, entry q
  auto state_index = [&](int i, int q) { return (16 * ph + lr) * N + 16 * (nb0 + NBS * i) + 4 * lq + q; };
  __shared__ unsigned sWord;

  // Chunks kb .. ke-1 of the current unit, from the state in hacc (staged in
  // LDS).  With a stop flag, the run also ends after a chunk once at least
  // k_stop chunks are done and the flag is set (thread 0 polls it, the
  // workgroup reads it through LDS); returns the first chunk not done.
  // (wavefront 0) the steps of the chunk at token t0 from the raw values in
  // graw, and their cumulative sum times A, into parity buffer `par`
  auto steps = [&](int t0, int par) {
    const float xv = graw + biash;
    float dl = p.softplus ? softplus_f(xv) : xv;
    dl = (t0 + lane < L) ? dl : 0.0f;  // past the end: no step, no input
    float cs = dl * Ah;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float up = __shfl_up(cs, o, 64);
      cs += lane >= o ? up : 0.0f;
    }
    sDL[par][lane] = dl;
    sCS[par][lane] = cs;
  };
  auto run_chunks = [&](int kb, int ke, const unsigned* stop_flag, int k_stop) -> int {
  if (ke <= kb) return kb;
  load_c(kb * Q);
  load_b(kb * Q);
  load_x(kb * Q);
  if (w == 0) steps(kb * Q, kb & 1);
  for (int k = kb; k < ke; ++k) {
    const int t0 = k * Q;
    const int par = k & 1;
    // ---- stage: C and B by token row, x transposed (the steps are ready in parity buffer par)
#pragma unroll
    for (int i = 0; i < C_PER; ++i) {
      const int e = tid + NTH * i;
      if (e < C_PIECES) *reinterpret_cast<u32x4_t*>(&sC[(e / (N / 8)) * SN + (e % (N / 8)) * 8]) = gc[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int e = tid + NTH * i;
      if (e < B_ITEMS) {
        const int np = e % (N / 2), s0 = 4 * (e / (N / 2));
#pragma unroll
        for (int r = 0; r < 4; ++r) *reinterpret_cast<uint32_t*>(&sB[(s0 + r) * SN + 2 * np]) = gb[i][r];
      }
    }
    if (tid < XI) {
      // x^T: channel 2xpp takes the low halves of the four rows, 2xpp+1 the high halves
      const u32x2_t even = {(gx[0] & 0xffffu) | (gx[1] << 16), (gx[2] & 0xffffu) | (gx[3] << 16)};
      const u32x2_t odd = {(gx[0] >> 16) | (gx[1] & 0xffff0000u), (gx[2] >> 16) | (gx[3] & 0xffff0000u)};
      *reinterpret_cast<u32x2_t*>(&sXT[(2 * xpp) * SQ + xs0]) = even;
      *reinterpret_cast<u32x2_t*>(&sXT[(2 * xpp + 1) * SQ + xs0]) = odd;
      if (p.z) {
        *reinterpret_cast<u32x2_t*>(&sZT[(2 * xpp) * SQ + xs0]) =
            u32x2_t{(gzz[0] & 0xffffu) | (gzz[1] << 16), (gzz[2] & 0xffffu) | (gzz[3] << 16)};
        *reinterpret_cast<u32x2_t*>(&sZT[(2 * xpp + 1) * SQ + xs0]) =
            u32x2_t{(gzz[0] >> 16) | (gzz[1] & 0xffff0000u), (gzz[2] >> 16) | (gzz[3] & 0xffff0000u)};
      }
    }
    __syncthreads();
    if (k + 1 < ke) {  // in flight through the chunk's products
      load_c(t0 + Q);
      load_x(t0 + Q);
    }

    // ---- Y (inter-chunk part) = C H for token block ty, channel blocks py0.. (from the state
    // staged at the end of the last chunk).  Issued ahead of the M and W work below, which does
    // not depend on it, so that the matrix cores run under that vector work.
    f32x4_t yacc[YT];
#pragma unroll
    for (int c = 0; c < YT; ++c) yacc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < N / 32; ++kk) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sC[(16 * ty + lr) * SN + 32 * kk + 8 * lq]);
#pragma unroll
      for (int c = 0; c < YT; ++c) {
        const int pr = (16 * (py0 + c) + lr) * SN + 32 * kk + 8 * lq;
        const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&sHh[pr]);
        const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&sHl[pr]);
        yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, yacc[c], 0, 0, 0);
        yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, yacc[c], 0, 0, 0);
      }
    }

    // ---- M[t][s] = G[t][s] exp(cs_t - cs_s) delta_s on s <= t, from tiles of G^T = B C^T on or
    // below the diagonal (wavefronts 0 and 1 take two of the ten, the others one), and zero for the
    // two tiles above it that the Y products read
    for (int gi = w; gi < 12; gi += NW) {
      int gs, gt;
      if (gi < 4) {
        gs = 0;
        gt = gi;
      } else if (gi < 7) {
        gs = 1;
        gt = gi - 3;
      } else if (gi < 9) {
        gs = 2;
        gt = gi - 5;
      } else if (gi < 10) {
        gs = 3;
        gt = 3;
      } else {
        gs = gi == 10 ? 1 : 3;
        gt = gs - 1;
      }
      const int t = 16 * gt + lr, s0 = 16 * gs + 4 * lq;
      float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (gi < 10) {
        f32x4_t g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < N / 32; ++kk) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sB[(16 * gs + lr) * SN + 32 * kk + 8 * lq]);
          const bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&sC[(16 * gt + lr) * SN + 32 * kk + 8 * lq]);
          g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, g, 0, 0, 0);
        }
        const float cst = sCS[par][t];
        const f32x4_t css = *reinterpret_cast<const f32x4_t*>(&sCS[par][s0]);
        const f32x4_t dls = *reinterpret_cast<const f32x4_t*>(&sDL[par][s0]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          m[j] = (s0 + j <= t) ? g[j] * __builtin_amdgcn_exp2f((cst - css[j]) * kLog2eF) * dls[j] : 0.0f;
      }
      u32x2_t hi, lo;
      split4(m, hi, lo);
      *reinterpret_cast<u32x2_t*>(&sMh[t * SQ + s0]) = hi;
      *reinterpret_cast<u32x2_t*>(&sMl[t * SQ + s0]) = lo;
    }
    // ---- W^T[n][s] = exp(cs_end - cs_s) delta_s B[s][n], from the B rows in registers
    {
      const float cse = sCS[par][Q - 1];
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        const int e = tid + NTH * i;
        if (e < B_ITEMS) {
          const int np = e % (N / 2), s0 = 4 * (e / (N / 2));
          const f32x4_t css = *reinterpret_cast<const f32x4_t*>(&sCS[par][s0]);
          const f32x4_t dls = *reinterpret_cast<const f32x4_t*>(&sDL[par][s0]);
          float v0[4], v1[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ws = __builtin_amdgcn_exp2f((cse - css[r]) * kLog2eF) * dls[r];
            v0[r] = ws * bf16_lo_of(gb[i][r]);
            v1[r] = ws * bf16_hi_of(gb[i][r]);
          }
          u32x2_t hi, lo;
          split4(v0, hi, lo);
          *reinterpret_cast<u32x2_t*>(&sWh[(2 * np) * SQ + s0]) = hi;
          *reinterpret_cast<u32x2_t*>(&sWl[(2 * np) * SQ + s0]) = lo;
          split4(v1, hi, lo);
          *reinterpret_cast<u32x2_t*>(&sWh[(2 * np + 1) * SQ + s0]) = hi;
          *reinterpret_cast<u32x2_t*>(&sWl[(2 * np + 1) * SQ + s0]) = lo;
        }
      }
    }
    __syncthreads();
    if (k + 1 < ke) load_b(t0 + Q);

    // ---- Y = exp(cs_t) C H + M x  (token block ty, channel blocks py0, py0+1), then the epilogue
    {
      const f32x4_t cst = *reinterpret_cast<const f32x4_t*>(&sCS[par][16 * ty + 4 * lq]);
#pragma unroll
      for (int c = 0; c < YT; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) yacc[c][j] *= __builtin_amdgcn_exp2f(cst[j] * kLog2eF);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (32 * kk > 16 * ty + 15) continue;  // M is zero past the diagonal
        const int mr = (16 * ty + lr) * SQ + 32 * kk + 8 * lq;
        const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&sMh[mr]);
        const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&sMl[mr]);
#pragma unroll
        for (int c = 0; c < YT; ++c) {
          const bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&sXT[(16 * (py0 + c) + lr) * SQ + 32 * kk + 8 * lq]);
          yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb, yacc[c], 0, 0, 0);
          yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb, yacc[c], 0, 0, 0);
        }
      }
      // + D x, times SiLU(z), rounded to bf16; x of four consecutive tokens is one 8-byte read of x^T
#pragma unroll
      for (int c = 0; c < YT; ++c) {
        const int pch = 16 * (py0 + c) + lr;
        const u32x2_t xq = *reinterpret_cast<const u32x2_t*>(&sXT[pch * SQ + 16 * ty + 4 * lq]);
        const float xv[4] = {bf16_lo_of(xq[0]), bf16_hi_of(xq[0]), bf16_lo_of(xq[1]), bf16_hi_of(xq[1])};
        u32x2_t zq = {0u, 0u};
        if (p.z) zq = *reinterpret_cast<const u32x2_t*>(&sZT[pch * SQ + 16 * ty + 4 * lq]);
        const float zv[4] = {bf16_lo_of(zq[0]), bf16_hi_of(zq[0]), bf16_lo_of(zq[1]), bf16_hi_of(zq[1])};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * ty + 4 * lq + j;
          float v = __builtin_fmaf(Dh, xv[j], yacc[c][j]);
          if (p.z) v *= silu_f(zv[j]);
          __builtin_amdgcn_raw_buffer_store_b16(bf16_bits_of(v), rs_y, ((t0 + t) * rowe + pch) * 2,
                                                0, 0);
        }
      }
    }

    // ---- H = exp(cs_end) H + W^T x  (channel block ph, state blocks nb0 + NBS i)
    {
      const float fade = __builtin_amdgcn_exp2f(sCS[par][Q - 1] * kLog2eF);
#pragma unroll
      for (int i = 0; i < HT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) hacc[i][j] *= fade;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&sXT[(16 * ph + lr) * SQ + 32 * kk + 8 * lq]);
#pragma unroll
        for (int i = 0; i < HT; ++i) {
          const int wr = (16 * (nb0 + NBS * i) + lr) * SQ + 32 * kk + 8 * lq;
          const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&sWh[wr]);
          const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&sWl[wr]);
          hacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb, hacc[i], 0, 0, 0);
          hacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb, hacc[i], 0, 0, 0);
        }
      }
    }
    if (w == 0 && k + 1 < ke) steps(t0 + Q, par ^ 1);  // the next chunk's raw steps arrived meanwhile
    __syncthreads();  // every read of H^T, x^T, W^T, C, B and M for this chunk is done
    stage_state();      // H^T for the next chunk
    if (stop_flag != nullptr && k + 1 - kb >= k_stop && k + 1 < ke) {
      if (tid == 0) sWord = __hip_atomic_load(stop_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const bool stop = sWord != 0u;
      __syncthreads();  // every wavefront has read the word before it is written again
      if (stop) return k + 1;
    }
  }
  return ke;
  };
  auto write_final = [&]() {
    if (p.final_state) {
      float* fs = p.final_state + ((b * H + h) * P) * N;
#pragma unroll
      for (int i = 0; i < HT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) fs[state_index(i, q)] = hacc[i][q];
    }
  };

  const int nchunks = static_cast<int>((L + Q - 1) / Q);
  // Which unit and chunks this workgroup runs, as up to three phases that
  // share one copy of the chunk loop:
  //   one workgroup per unit:  phase 2 only, unit blockIdx.x, all chunks;
  //   chained, ticket j:       phase 0 (segment sg > 0 only): unit j from its
  //                            start until segment sg-1 has handed on its state
  //                            (after at least sg segment-lengths);
  //                            phase 1 (left-over units only): segment sg of
  //                            unit n_long + st, from the state handed on;
  //                            phase 2: unit j, the rest.
  // Segment 0 goes first; the whole unit's state waits in registers meanwhile.
  int j = static_cast<int>(blockIdx.x), sg = 0, st = 0;
  bool has_seg = false;
  if (p.n_split > 0) {
    if (tid == 0) sWord = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    j = static_cast<int>(__builtin_amdgcn_readfirstlane(sWord));
    __syncthreads();
    has_seg = j < p.n_split * p.Ks;
    sg = has_seg ? j / p.n_split : 0;
    st = has_seg ? j % p.n_split : 0;
  }
  const int seg_chunks = static_cast<int>(p.seg_chunks);
  const int kb = sg * seg_chunks < nchunks ? sg * seg_chunks : nchunks;
  const int ke = (sg + 1) * seg_chunks < nchunks ? (sg + 1) * seg_chunks : nchunks;
  unsigned* my_flag = has_seg ? p.flags + static_cast<int64_t>(st) * p.Ks + sg : nullptr;  // set once sg-1 is done
  float* crow = has_seg ? p.carry + (static_cast<int64_t>(st) * p.Ks + sg) * P * N : nullptr;  // [n_split][Ks][P][N]
  // the state of unit `unit` before its token 0: zero, or the given one
  auto initial = [&](int unit, f32x4_t* dst) {
#pragma unroll
    for (int i = 0; i < HT; ++i) {
      dst[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (p.h0) {
        const float* src = p.h0 + static_cast<int64_t>(unit) * P * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[i][q] = src[state_index(i, q)];
      }
    }
  };
  // unit j's starting state, kept here while a segment runs first (phase 0)
  f32x4_t saved[HT];
  int rest = 0;
  initial(j, saved);
  for (int phase = 0; phase < 3; ++phase) {
    if (phase == 0 && !(has_seg && sg > 0)) continue;
    if (phase == 1 && !has_seg) continue;
    // ---- before the phase: the unit and its starting state (a segment past the first takes its state
    // from the segment before it, below)
    set_unit(phase == 1 ? p.n_long + st : j);
    if (phase == 1) {
      initial(p.n_long + st, hacc);
    } else {
#pragma unroll
      for (int i = 0; i < HT; ++i) hacc[i] = saved[i];
    }
    if (phase == 1 && sg > 0) {
      // the state after segment sg-1: wait for its flag, then read it coherently
      if (tid == 0) {
        unsigned polls = 0;
        while (__hip_atomic_load(my_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
          if (++polls > kSsdSpinLimit) {
            __hip_atomic_fetch_or(p.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
      }
      __syncthreads();
      const bool lost = __hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
#pragma unroll
      for (int i = 0; i < HT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          hacc[i][q] = lost ? __builtin_nanf("")
                            : __hip_atomic_load(crow + state_index(i, q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    stage_state();
    const int r = run_chunks(phase == 0 ? 0 : (phase == 1 ? kb : rest), phase == 1 ? ke : nchunks,
                             phase == 0 ? my_flag : nullptr, phase == 0 ? sg * seg_chunks : 0);
    // ---- after the phase
    if (phase == 0) {
      rest = r;
#pragma unroll
      for (int i = 0; i < HT; ++i) saved[i] = hacc[i];
    } else if (phase == 1 && sg + 1 < p.Ks) {
      float* next = crow + P * N;
#pragma unroll
      for (int i = 0; i < HT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __hip_atomic_store(next + state_index(i, q), hacc[i][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(kSsdWaitVm0);  // this thread's carry stores have completed
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(p.flags + static_cast<int64_t>(st) * p.Ks + sg + 1, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      write_final();
    }
  }
}

}  // namespace ssm
