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
// chunk (v_mfma_f32_16x16x32_f16, fp32 accumulation):
//   G^T = B C^T              (Q x Q, K = N) -> M[t][s] = G[t][s] exp(cs_t - cs_s) delta_s on s <= t
//   Y   = exp(cs_t) C H + M x  (Q x P; K = N, then K = Q)  -> + D x, times SiLU(z), y
//   H   = exp(cs_end) H + W^T x   (N x P, K = Q),  W[s][n] = exp(cs_end - cs_s) delta_s B[s][n]
// C, B (by token row), M (by output row) and H^T [p][n] sit in LDS with their
// K index contiguous, so a fragment is one 16-byte read; the accumulators of
// G^T and H hold four consecutive K-side indices per lane, so M and H^T are
// written as 8-byte runs.  x, z and W, whose K index is the token, are stored
// by token row as they arrive (x [s][p], z [t][p], W [s][n]: consecutive lanes
// write consecutive columns of one row, free of bank conflicts) and read with
// gfx950's transposed LDS read (ds_read_b64_tr_b16), which hands each lane
// four consecutive tokens of one column.  (Writing them transposed instead put
// the 64 lanes of a store on rows two apart, eight banks for 128 dwords.)
//
// Two barriers per chunk: C and B are staged before the first; x, z, C H, M
// and W between the two; M x, the epilogue, the state update and the staging
// of the next state after the second, from where each wavefront goes straight
// on to the next chunk's C and B (no operand that this last part reads is
// rewritten before the next chunk's first barrier).
//
// Precision.  B, C and x arrive as bf16 and are staged as fp16, exactly
// (every bf16 value of magnitude 2^-14 .. 65504 is an fp16 value), so G^T =
// B C^T is exact.  The products take fp16 operands (11 significant bits,
// fp32 accumulation): M and the state H^T are rounded
// to fp16 once (relative 2^-12), which leaves y at the rounding of its own
// bf16 store (~4e-3); W, which carries every input into the state, is a pair
// hi + lo of fp16 (22 significant bits) entering its product as two MFMAs, so
// the state keeps its fp32 accuracy (~2e-5).  x, C, M, W and H must stay
// below 65504 in magnitude (the fp16 range); larger values give inf/NaN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ssm {

struct SsdParams {
  const void* x;       // [batch][L][H][P] bf16
  const void* delta;   // [batch][L][H] bf16 (raw)
  const float* A;      // [H]
  const void* B;       // [batch][L][ngroups][N] bf16
  const void* C;       // [batch][L][ngroups][N] bf16
  const float* D;      // [H] (nullable)
  const void* z;       // [batch][L][H][P] bf16 (nullable)
  const float* bias;   // [H] (nullable)
  void* y;             // [batch][L][H][P] bf16
  float* final_state;  // [batch][H][P][N] (nullable)
  const float* h0;     // [batch][H][P][N]: the state before token 0 (nullable: zero)
  int64_t batch, L, H;
  int64_t ngroups;     // head h reads group h / (H / ngroups) of B and C
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
  unsigned spin_limit;             // polls per wait (poll_ready)
  const unsigned* wait_override;   // test hook: a word no one sets, polled instead of every flag
};

// A chained segment waits for the state handed on to it with poll_ready; past
// the limit it sets the status word and goes on from a NaN state, so the
// kernel always ends and the outputs that depend on the lost hand-off show the
// failure.
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
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned short bf16_bits_of(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_value(unsigned short b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
__device__ __forceinline__ float bf16_lo_of(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi_of(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Four fp32 values rounded to fp16 (nearest even), packed as one 8-byte run; and as a pair hi + lo of fp16
// runs (hi = fp16(v), lo = fp16(v - hi)), 22 significant bits.
__device__ __forceinline__ u32x2_t cvt4_f16(const float* v) {
  const f16x4_t h = __builtin_convertvector((f32x4_t){v[0], v[1], v[2], v[3]}, f16x4_t);
  return __builtin_bit_cast(u32x2_t, h);
}
__device__ __forceinline__ void split4_f16(const float* v, u32x2_t& hi, u32x2_t& lo) {
  const f32x4_t x = {v[0], v[1], v[2], v[3]};
  const f16x4_t h = __builtin_convertvector(x, f16x4_t);
  const f16x4_t l = __builtin_convertvector(x - __builtin_convertvector(h, f32x4_t), f16x4_t);
  hi = __builtin_bit_cast(u32x2_t, h);
  lo = __builtin_bit_cast(u32x2_t, l);
}
// bf16 values as fp16 (exact for |v| in [2^-14, 65504]: every bf16 value there has at most 8 significant bits),
// two per 32-bit word and eight per 16-byte piece.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const f16x2_t h = __builtin_convertvector((f32x2_t){__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)},
                                            f16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ u32x4_t bf16x8_to_f16(u32x4_t v) {
  return u32x4_t{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
}
__device__ __forceinline__ float f16_lo_of(uint32_t pair) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(pair & 0xffffu)));
}
__device__ __forceinline__ float f16_hi_of(uint32_t pair) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(pair >> 16)));
}

// Transposed LDS read (ds_read_b64_tr_b16, gfx950).  Within each group of 16
// lanes, lane i returns, as element j, the 16-bit value that lane 4j + i/4 of
// its group addresses at position i % 4 of its own 8-byte run.  So if lane
// (g, i) of group g addresses row r0(g) + i/4 of a row-major array at column
// c0 + 4 (i % 4), lane (g, i) receives column c0 + i of rows r0(g) .. r0(g)+3:
// four consecutive K values of one MFMA row or column, from an array stored
// with K as its row index.  row_of / col_of give that addressing.
__device__ __forceinline__ u32x2_t lds_read_tr4(const unsigned short* base, int row0, int col0, int stride) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const int i = threadIdx.x & 15;
  const unsigned short* a = base + (row0 + (i >> 2)) * stride + col0 + 4 * (i & 3);
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a));
  return __builtin_bit_cast(u32x2_t, v);
}
// An MFMA 16x16x32 operand fragment from a row-major [K][.] array (K rows k0 .. k0+31, column col0 + lr): two
// transposed reads.  Lane group lq takes K rows k0 + 4 lq .. k0 + 4 lq + 3 and k0 + 16 + 4 lq .. k0 + 16 + 4 lq + 3,
// not 8 lq .. 8 lq + 7: the two groups of 16 lanes that a read serves together then touch 8 consecutive rows,
// which lie on distinct banks.  The contraction does not depend on the order of K as long as both operands of a
// product share it: the other operand is a fragment from here too, or M, whose columns are stored in this order
// (kperm_col).
__device__ __forceinline__ f16x8_t lds_frag_tr(const unsigned short* base, int k0, int col0, int lq, int stride) {
  const u32x2_t a = lds_read_tr4(base, k0 + 4 * lq, col0, stride);
  const u32x2_t b = lds_read_tr4(base, k0 + 16 + 4 * lq, col0, stride);
  return __builtin_bit_cast(f16x8_t, u32x4_t{a[0], a[1], b[0], b[1]});
}
// Where the run of four K indices starting at k (a multiple of 4) is stored in a row whose 16-byte fragment
// reads must follow lds_frag_tr's K order: run j of a 32-wide block goes to position 2 j (j < 4) or 2 (j - 4) + 1.
__device__ __forceinline__ int kperm_col(int k) {
  const int j = (k >> 2) & 7;
  return (k & ~31) + 4 * (j < 4 ? 2 * j : 2 * (j - 4) + 1);
}

template <int N>
__global__ void __launch_bounds__(64 * ssd_waves(N)) ssd_kernel(SsdParams p) {
  constexpr int Q = kSsdQ, P = kSsdP, NW = ssd_waves(N), NTH = 64 * NW;
  static_assert(N == 32 || N == 64 || N == 128, "dstate: 32, 64 or 128");
  constexpr int SN = N + 8;  // padded rows (elements) of the [.][N] arrays: 16-byte aligned, banks staggered
  constexpr int SQ = Q + 8;  // padded rows of the [.][Q] arrays
  // Rows of the arrays read transposed (x, z by channel, W by state): a row is (8 x odd) dwords, so the 16
  // rows x 32 bytes that a transposed read of 64 lanes touches cover every bank four times, and the row
  // writes (one token row, consecutive lanes on consecutive columns) are conflict-free.
  constexpr int SX = P + 16;
  constexpr int SW = N + 16;
  constexpr int NT = N / 16;  // 16-wide state tiles
  constexpr int HT = NT * 4 / NW;  // state tiles per wavefront (NT x 4 tiles over NW wavefronts)
  constexpr int YT = 16 / NW;      // Y tiles per wavefront (4 x 4 over NW wavefronts)
  constexpr int XR = Q * (P / 2) / NTH;  // token rows of a thread's x item (two channels of XR consecutive rows)
  constexpr int C_PIECES = Q * N / 8;         // 16-byte pieces of a chunk's C
  constexpr int C_PER = (C_PIECES + NTH - 1) / NTH;
  constexpr int B_ITEMS = (Q / 4) * (N / 2);  // (4 tokens) x (2 states) items of a chunk's B
  constexpr int B_PER = (B_ITEMS + NTH - 1) / NTH;
  static_assert(XR >= 1 && XR * NTH == Q * (P / 2) && HT >= 1 && YT >= 1, "work split");
  constexpr float kLog2eF = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) unsigned short sC[Q * SN];   // C [t][n], fp16
  __shared__ __attribute__((aligned(16))) unsigned short sB[Q * SN];   // B [s][n], fp16
  __shared__ __attribute__((aligned(16))) unsigned short sWh[Q * SW];  // W [s][n], fp16 hi
  __shared__ __attribute__((aligned(16))) unsigned short sWl[Q * SW];  // fp16 lo
  __shared__ __attribute__((aligned(16))) unsigned short sX[Q * SX];   // x [s][p], fp16
  __shared__ __attribute__((aligned(16))) unsigned short sZ[Q * SX];   // z [t][p], bf16
  __shared__ __attribute__((aligned(16))) unsigned short sM[Q * SQ];   // M [t][s], fp16
  __shared__ __attribute__((aligned(16))) unsigned short sH[P * SN];   // H^T [p][n], fp16
  // per chunk parity: A * (cumulative step) within the chunk, and the step delta_t; wavefront 0
  // prepares the next chunk's while the others finish the current one
  __shared__ __attribute__((aligned(16))) float sCS[2][Q];
  __shared__ __attribute__((aligned(16))) float sDL[2][Q];
  // and per token, once: exp(cs_t) (the inter-chunk readout's fade) and exp(cs_end - cs_s) delta_s (the
  // weight of token s in the state update)
  __shared__ __attribute__((aligned(16))) float sECS[2][Q];
  __shared__ __attribute__((aligned(16))) float sWS[2][Q];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t H = p.H, L = p.L;
  // elements between token rows of x, z, y; the host keeps every token-row
  // byte offset (one chunk past L included) below 2^31, so offsets are 32-bit
  const int rowe = static_cast<int>(H * P);
  const int H32 = static_cast<int>(H);
  const int BS = static_cast<int>(p.ngroups) * N;  // elements per token row of B and C

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
    // B and C of the head's group: token rows of BS elements, the group's N at offset g * N
    const int64_t g = h / (H / p.ngroups);
    const int64_t bcbase = (b * L * p.ngroups + g) * N;
    rs_b = make_rsrc(static_cast<const unsigned short*>(p.B) + bcbase, (L * p.ngroups - g) * N * 2);
    rs_c = make_rsrc(static_cast<const unsigned short*>(p.C) + bcbase, (L * p.ngroups - g) * N * 2);
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
  uint32_t gb[B_PER][4], gx[XR], gzz[XR];
  float graw = 0.0f;
  auto load_c = [&](int t0) {
#pragma unroll
    for (int i = 0; i < C_PER; ++i) {
      const int e = tid + NTH * i;
      const int row = e / (N / 8), col = (e % (N / 8)) * 8;
      if (e < C_PIECES)
        gc[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rs_c, ((t0 + row) * BS + col) * 2, 0, 0));
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
          gb[i][r] = __builtin_amdgcn_raw_buffer_load_b32(rs_b, ((t0 + s0 + r) * BS + 2 * np) * 2, 0, 0);
      }
    }
  };
  // x item of every thread: channels 2xpp, 2xpp+1 of tokens xs0 .. xs0+XR-1
  const int xpp = tid % (P / 2), xs0 = XR * (tid / (P / 2));
  auto load_x = [&](int t0) {
    {
#pragma unroll
      for (int r = 0; r < XR; ++r)
        gx[r] = __builtin_amdgcn_raw_buffer_load_b32(rs_x, ((t0 + xs0 + r) * rowe + 2 * xpp) * 2, 0, 0);
      if (p.z) {
#pragma unroll
        for (int r = 0; r < XR; ++r)
          gzz[r] = __builtin_amdgcn_raw_buffer_load_b32(rs_z, ((t0 + xs0 + r) * rowe + 2 * xpp) * 2, 0, 0);
      }
    }
    if (w == 0)
      graw = bf16_value(static_cast<unsigned short>(__builtin_amdgcn_raw_buffer_load_b16(
          rs_d, (t0 + lane) * H32 * 2, 0, 0)));
  };
  f32x4_t hacc[HT];
  // H^T in fp16 for the Y products, from the accumulators: four
  // consecutive states of one channel per lane (this wavefront's tiles only)
  auto stage_state = [&]() {
#pragma unroll
    for (int i = 0; i < HT; ++i) {
      const float v[4] = {hacc[i][0], hacc[i][1], hacc[i][2], hacc[i][3]};
      const int idx = (16 * ph + lr) * SN + 16 * (nb0 + NBS * i) + 4 * lq;
      *reinterpret_cast<u32x2_t*>(&sH[idx]) = cvt4_f16(v);
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
  // graw, their cumulative sum times A, and the fades that depend on one token
  // only, into parity buffer `par`
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
    const float cse = __shfl(cs, Q - 1, 64);
    sDL[par][lane] = dl;
    sCS[par][lane] = cs;
    sECS[par][lane] = __builtin_amdgcn_exp2f(cs * kLog2eF);
    sWS[par][lane] = __builtin_amdgcn_exp2f((cse - cs) * kLog2eF) * dl;
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
      if (e < C_PIECES) *reinterpret_cast<u32x4_t*>(&sC[(e / (N / 8)) * SN + (e % (N / 8)) * 8]) = bf16x8_to_f16(gc[i]);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int e = tid + NTH * i;
      if (e < B_ITEMS) {
        const int np = e % (N / 2), s0 = 4 * (e / (N / 2));
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<uint32_t*>(&sB[(s0 + r) * SN + 2 * np]) = bf16x2_to_f16x2(gb[i][r]);
      }
    }
    __syncthreads();
    // x as fp16 and z as loaded, by token row (channels 2xpp, 2xpp+1 of rows xs0 .. xs0+3).  They are first read
    // after the next barrier, and the last chunk's reads of them ended before the one above, so staging them
    // here spares a barrier at the end of the chunk.
    {
#pragma unroll
      for (int r = 0; r < XR; ++r) *reinterpret_cast<uint32_t*>(&sX[(xs0 + r) * SX + 2 * xpp]) = bf16x2_to_f16x2(gx[r]);
      if (p.z) {
#pragma unroll
        for (int r = 0; r < XR; ++r) *reinterpret_cast<uint32_t*>(&sZ[(xs0 + r) * SX + 2 * xpp]) = gzz[r];
      }
    }
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
      const f16x8_t a = *reinterpret_cast<const f16x8_t*>(&sC[(16 * ty + lr) * SN + 32 * kk + 8 * lq]);
#pragma unroll
      for (int c = 0; c < YT; ++c) {
        const int pr = (16 * (py0 + c) + lr) * SN + 32 * kk + 8 * lq;
        const f16x8_t bh = *reinterpret_cast<const f16x8_t*>(&sH[pr]);
        yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, yacc[c], 0, 0, 0);
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
          const f16x8_t a = *reinterpret_cast<const f16x8_t*>(&sB[(16 * gs + lr) * SN + 32 * kk + 8 * lq]);
          const f16x8_t bb = *reinterpret_cast<const f16x8_t*>(&sC[(16 * gt + lr) * SN + 32 * kk + 8 * lq]);
          g = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bb, g, 0, 0, 0);
        }
        const float cst = sCS[par][t];
        const f32x4_t css = *reinterpret_cast<const f32x4_t*>(&sCS[par][s0]);
        const f32x4_t dls = *reinterpret_cast<const f32x4_t*>(&sDL[par][s0]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          m[j] = (s0 + j <= t) ? g[j] * __builtin_amdgcn_exp2f((cst - css[j]) * kLog2eF) * dls[j] : 0.0f;
      }
      *reinterpret_cast<u32x2_t*>(&sM[t * SQ + kperm_col(s0)]) = cvt4_f16(m);  // in lds_frag_tr's K order
    }
    // ---- W[s][n] = exp(cs_end - cs_s) delta_s B[s][n], from the B rows in registers, by token row
    {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        const int e = tid + NTH * i;
        if (e < B_ITEMS) {
          const int np = e % (N / 2), s0 = 4 * (e / (N / 2));
          const f32x4_t ws = *reinterpret_cast<const f32x4_t*>(&sWS[par][s0]);
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) {
            // rows s0 + 2 r2 and s0 + 2 r2 + 1: four values, split as hi + lo
            const float v[4] = {ws[2 * r2] * bf16_lo_of(gb[i][2 * r2]), ws[2 * r2] * bf16_hi_of(gb[i][2 * r2]),
                                ws[2 * r2 + 1] * bf16_lo_of(gb[i][2 * r2 + 1]),
                                ws[2 * r2 + 1] * bf16_hi_of(gb[i][2 * r2 + 1])};
            u32x2_t hi, lo;
            split4_f16(v, hi, lo);
            *reinterpret_cast<uint32_t*>(&sWh[(s0 + 2 * r2) * SW + 2 * np]) = hi[0];
            *reinterpret_cast<uint32_t*>(&sWl[(s0 + 2 * r2) * SW + 2 * np]) = lo[0];
            *reinterpret_cast<uint32_t*>(&sWh[(s0 + 2 * r2 + 1) * SW + 2 * np]) = hi[1];
            *reinterpret_cast<uint32_t*>(&sWl[(s0 + 2 * r2 + 1) * SW + 2 * np]) = lo[1];
          }
        }
      }
    }
    __syncthreads();
    if (k + 1 < ke) load_b(t0 + Q);

    // ---- Y = exp(cs_t) C H + M x  (token block ty, channel blocks py0, py0+1), then the epilogue
    {
      const f32x4_t ecs = *reinterpret_cast<const f32x4_t*>(&sECS[par][16 * ty + 4 * lq]);
#pragma unroll
      for (int c = 0; c < YT; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) yacc[c][j] *= ecs[j];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (32 * kk > 16 * ty + 15) continue;  // M is zero past the diagonal
        const int mr = (16 * ty + lr) * SQ + 32 * kk + 8 * lq;
        const f16x8_t ah = *reinterpret_cast<const f16x8_t*>(&sM[mr]);
#pragma unroll
        for (int c = 0; c < YT; ++c) {
          const f16x8_t bb = lds_frag_tr(sX, 32 * kk, 16 * (py0 + c), lq, SX);
          yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bb, yacc[c], 0, 0, 0);
        }
      }
      // + D x, times SiLU(z), rounded to bf16; x and z of four consecutive tokens are one transposed read each
#pragma unroll
      for (int c = 0; c < YT; ++c) {
        const int pch = 16 * (py0 + c) + lr;
        const u32x2_t xq = lds_read_tr4(sX, 16 * ty + 4 * lq, 16 * (py0 + c), SX);
        const float xv[4] = {f16_lo_of(xq[0]), f16_hi_of(xq[0]), f16_lo_of(xq[1]), f16_hi_of(xq[1])};
        u32x2_t zq = {0u, 0u};
        if (p.z) zq = lds_read_tr4(sZ, 16 * ty + 4 * lq, 16 * (py0 + c), SX);
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
      const float fade = sECS[par][Q - 1];
#pragma unroll
      for (int i = 0; i < HT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) hacc[i][j] *= fade;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f16x8_t bb = lds_frag_tr(sX, 32 * kk, 16 * ph, lq, SX);
#pragma unroll
        for (int i = 0; i < HT; ++i) {
          const f16x8_t ah = lds_frag_tr(sWh, 32 * kk, 16 * (nb0 + NBS * i), lq, SW);
          const f16x8_t al = lds_frag_tr(sWl, 32 * kk, 16 * (nb0 + NBS * i), lq, SW);
          hacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bb, hacc[i], 0, 0, 0);
          hacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bb, hacc[i], 0, 0, 0);
        }
      }
    }
    if (w == 0 && k + 1 < ke) steps(t0 + Q, par ^ 1);  // the next chunk's raw steps arrived meanwhile
    // No barrier here: the next chunk's C and B (staged next) and H^T are not read in this part of the chunk, and
    // its M, W, x and z are written only after the next chunk's first barrier.
    stage_state();      // H^T for the next chunk (read after the next chunk's first barrier)
    if (stop_flag != nullptr && k + 1 - kb >= k_stop && k + 1 < ke) {
      if (tid == 0) sWord = __hip_atomic_load(stop_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const bool stop = sWord != 0u;
      __syncthreads();  // every wavefront has read the word before it is written again
      if (stop) return k + 1;
    }
  }
  __syncthreads();  // every read of this run's operands is done before the caller stages anything
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
  // set once segment sg-1 is done
  const unsigned* my_flag =
      has_seg ? (p.wait_override ? p.wait_override : p.flags + static_cast<int64_t>(st) * p.Ks + sg) : nullptr;
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
  // unit j's state while a segment runs (phase 1): each thread's own state tiles, kept in LDS rather than in
  // registers that would stay allocated through the chunk loop
  __shared__ f32x4_t sSaved[HT][NTH];
  int rest = 0;
  {
    f32x4_t s0[HT];
    initial(j, s0);
#pragma unroll
    for (int i = 0; i < HT; ++i) sSaved[i][tid] = s0[i];
  }
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
      for (int i = 0; i < HT; ++i) hacc[i] = sSaved[i][tid];
    }
    if (phase == 1 && sg > 0) {
      // the state after segment sg-1: wait for its flag, then read it coherently
      if (tid == 0) {
        const bool ok = poll_ready(my_flag, p.spin_limit);
        if (!ok) __hip_atomic_fetch_or(p.status, kStatusHandoffTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sWord = ok ? 1u : 0u;
      }
      __syncthreads();
      const bool lost = sWord == 0u;  // this wait ran out (not another's)
      __syncthreads();                // read by every wavefront before the word is written again
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
      for (int i = 0; i < HT; ++i) sSaved[i][tid] = hacc[i];
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
