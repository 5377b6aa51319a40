// ssd_kernel.hpp -- the Mamba-2 state-space-duality (SSD) layer on MFMA.
//
// Mamba-2 gives every head one scalar state matrix A (times the identity), so
// the sequence map of a head is multiplication by a causal 1-semiseparable
// matrix and can be computed blockwise with matrix products ("State Space
// Models and the Post-Transformer Era", "Mamba-2 and Structured State Space
// Duality"; "The State That Must Remember Everything", Part 4).  Per batch row
// and head (headdim P = 64 channels sharing delta_t and A, with B_t, C_t of
// dstate N shared by all heads) the state H (P x N) runs
//     H_t = exp(delta_t A) H_{t-1} + delta_t x_t B_t^T,   y_t = H_t C_t + D x_t,
// then y is gated by SiLU(z).  Over a chunk of Q tokens with
// cs_t = A (delta_0 + ... + delta_t) (chunk-local, inclusive) this is
//     y_t   = exp(cs_t) C_t . H_prev                                  (inter)
//           + sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) delta_s x_s        (intra)
//     H_end = exp(cs_end) H_prev + sum_s exp(cs_end - cs_s) delta_s x_s B_s^T.
//
// One workgroup (4 wavefronts) per (batch row, head) walks the chunks in
// order; the head's state stays in MFMA accumulators (fp32) the whole time,
// so no chunk states go to HBM and x, z, y, B, C are each read or written
// once.  Per chunk, with bf16 operands and fp32 accumulation
// (v_mfma_f32_16x16x32_bf16; wavefront w owns rows 16w..16w+15 of each product):
//   G   = C B^T                  (Q x Q, K = N)  -> M = G * exp(cs_t - cs_s) * delta_s on s <= t, to LDS
//   Y   = exp(cs_t) (C H^T^T)    (Q x P, K = N)  +  M x   (K = Q)   -> epilogue D x, SiLU(z), y
//   H^T = exp(cs_end) H^T + x^T W  (P x N, K = Q), W[s][n] = exp(cs_end - cs_s) delta_s B[s][n]
// Operands sit in LDS in the orientation whose K index is contiguous, so
// every fragment is one 16-byte read: C and B row-major, x, W and H
// transposed.  W takes the LDS of B once G is done.
//
// Precision.  C, B and x arrive as bf16 and are exact operands.  M, W and the
// state are fp32 values; rounded to bf16 once, the sums they enter lose
// about 2^-9 of their largest terms, which measured against the fp64 oracle
// puts y near 2e-2 of its scale.  Each of the three is therefore carried as a
// pair hi + lo of bf16 (hi = bf16(v), lo = bf16(v - hi), 16 significant bits)
// and enters its product as two MFMAs, which brings y to the rounding of its
// own bf16 store (~4e-3) and the state to ~2e-5.  The pairs take the
// workgroup to 115 KB of LDS, one per CU.
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
  int64_t batch, L, H;
  int softplus;
};

constexpr int kSsdQ = 64;  // tokens per chunk
constexpr int kSsdP = 64;  // channels per head

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned short bf16_bits_of(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_value(unsigned short b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

template <int N>
__global__ void __launch_bounds__(256) ssd_kernel(SsdParams p) {
  constexpr int Q = kSsdQ, P = kSsdP;
  static_assert(N % 32 == 0 && N <= 128, "dstate: a multiple of 32 up to 128");
  constexpr int SN = N + 8;  // padded rows (elements) of the [.][N] arrays: 16-byte aligned, banks staggered
  constexpr int SQ = Q + 8;  // padded rows of the [.][Q] arrays
  constexpr int BW = (Q * SN > N * SQ) ? Q * SN : N * SQ;
  constexpr int NT = N / 16;               // 16-wide state tiles
  constexpr int BC_PASSES = N / 32;        // 16-byte pieces of a chunk's B (or C) rows per thread
  constexpr float kLog2eF = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) unsigned short sC[Q * SN];   // C rows [t][n]
  __shared__ __attribute__((aligned(16))) unsigned short sB[BW];       // B rows [s][n], then W (hi) [n][s]
  __shared__ __attribute__((aligned(16))) unsigned short sWl[N * SQ];  // W (lo) [n][s]
  __shared__ __attribute__((aligned(16))) unsigned short sXT[P * SQ];  // x transposed [p][s]
  __shared__ __attribute__((aligned(16))) unsigned short sM[Q * SQ];   // masked, decayed C B^T (hi) [t][s]
  __shared__ __attribute__((aligned(16))) unsigned short sMl[Q * SQ];  // (lo)
  __shared__ __attribute__((aligned(16))) unsigned short sHT[P * SN];  // H^T (hi) [p][n]
  __shared__ __attribute__((aligned(16))) unsigned short sHl[P * SN];  // (lo)
  __shared__ __attribute__((aligned(16))) float sCS[Q];             // A * (cumulative step) within the chunk
  __shared__ float sDL[Q];                                             // the step delta_t

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t H = p.H, L = p.L;
  const int64_t b = blockIdx.x / H, h = blockIdx.x % H;
  const int64_t rowe = H * P;  // elements between token rows of x, z, y
  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.0f;
  const float biash = p.bias ? p.bias[h] : 0.0f;

  // Buffer resources: token rows past L read as zero and are not written.
  const int64_t xbase = (b * L * H + h) * P;
  const int64_t xbytes = (L * H - h) * P * 2;
  const rsrc_t rs_x = make_rsrc(static_cast<const unsigned short*>(p.x) + xbase, xbytes);
  const rsrc_t rs_z = make_rsrc(p.z ? static_cast<const unsigned short*>(p.z) + xbase : nullptr, p.z ? xbytes : 0);
  const rsrc_t rs_y = make_rsrc(static_cast<unsigned short*>(p.y) + xbase, xbytes);
  const rsrc_t rs_b = make_rsrc(static_cast<const unsigned short*>(p.B) + b * L * N, L * N * 2);
  const rsrc_t rs_c = make_rsrc(static_cast<const unsigned short*>(p.C) + b * L * N, L * N * 2);
  const rsrc_t rs_d = make_rsrc(static_cast<const unsigned short*>(p.delta) + b * L * H + h, (L * H - h) * 2);

  // Loads of one chunk: x (2 pieces of 8 channels of a token row per
  // thread), B and C (BC_PASSES pieces of 8 states), the raw step (one token per thread of wavefront 0).
  u32x4_t gx[2], gb[BC_PASSES], gc[BC_PASSES];
  float graw = 0.0f;
  const int xr = tid >> 3, xc = (tid & 7) * 8;                  // x piece: row xr (+32), channels xc..xc+7
  constexpr int BC_TPR = N / 8;                                  // threads per B/C row
  const int bcr = tid / BC_TPR, bcc = (tid % BC_TPR) * 8;        // B/C piece: row bcr (+256/BC_TPR), states bcc..
  constexpr int BC_RSTEP = 256 / BC_TPR;
  auto load_xc = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      gx[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs_x, static_cast<int>(((t0 + xr + 32 * i) * rowe + xc) * 2), 0, 0));
#pragma unroll
    for (int i = 0; i < BC_PASSES; ++i)
      gc[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs_c, static_cast<int>(((t0 + bcr + BC_RSTEP * i) * N + bcc) * 2), 0, 0));
    if (w == 0)
      graw = bf16_value(static_cast<unsigned short>(__builtin_amdgcn_raw_buffer_load_b16(
          rs_d, static_cast<int>((t0 + lane) * H * 2), 0, 0)));
  };
  auto load_b = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < BC_PASSES; ++i)
      gb[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs_b, static_cast<int>(((t0 + bcr + BC_RSTEP * i) * N + bcc) * 2), 0, 0));
  };

  // The state H^T [P x N]: wavefront w owns rows 16w..16w+15, NT tiles of 16 states.
  f32x4_t hacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) hacc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int e = tid; e < P * SN; e += 256) sHT[e] = sHl[e] = 0;

  const int64_t nchunks = (L + Q - 1) / Q;
  load_xc(0);
  load_b(0);
  for (int64_t k = 0; k < nchunks; ++k) {
    const int64_t t0 = k * Q;
    // ---- stage the chunk: C, B rows; x transposed; steps and their cumulative sums
#pragma unroll
    for (int i = 0; i < BC_PASSES; ++i) {
      *reinterpret_cast<u32x4_t*>(&sC[(bcr + BC_RSTEP * i) * SN + bcc]) = gc[i];
      *reinterpret_cast<u32x4_t*>(&sB[(bcr + BC_RSTEP * i) * SN + bcc]) = gb[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sXT[(xc + e) * SQ + xr + 32 * i] = static_cast<unsigned short>(gx[i][e / 2] >> (16 * (e % 2)));
    }
    if (w == 0) {
      const float xv = graw + biash;
      float dl = p.softplus ? softplus_f(xv) : xv;
      dl = (t0 + lane < L) ? dl : 0.0f;  // past the end: no step, no input
      float cs = dl * Ah;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float up = __shfl_up(cs, o, 64);
        cs += lane >= o ? up : 0.0f;
      }
      sDL[lane] = dl;
      sCS[lane] = cs;
    }
    __syncthreads();
    if (k + 1 < nchunks) load_xc(t0 + Q);  // in flight through the chunk's products

    // ---- M = (C B^T) * exp(cs_t - cs_s) * delta_s on s <= t (wavefront w: rows 16w..16w+15)
    {
      f32x4_t g[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) g[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sC[(16 * w + lr) * SN + 32 * kk + 8 * lq]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c > w) continue;  // wholly above the diagonal
          const bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&sB[(16 * c + lr) * SN + 32 * kk + 8 * lq]);
          g[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, g[c], 0, 0, 0);
        }
      }
      const f32x4_t cst = *reinterpret_cast<const f32x4_t*>(&sCS[16 * w + 4 * lq]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int s = 16 * c + lr;
        const float css = sCS[s], dls = sDL[s];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * w + 4 * lq + j;
          const float m = (s <= t) ? g[c][j] * __builtin_amdgcn_exp2f((cst[j] - css) * kLog2eF) * dls : 0.0f;
          const unsigned short hi = bf16_bits_of(m);
          sM[t * SQ + s] = hi;
          sMl[t * SQ + s] = bf16_bits_of(m - bf16_value(hi));
        }
      }
    }
    __syncthreads();

    // ---- W = exp(cs_end - cs_s) delta_s B[s][n], transposed into B's LDS (B's reads are done)
    {
      const float cse = sCS[Q - 1];
#pragma unroll
      for (int i = 0; i < BC_PASSES; ++i) {
        const int s = bcr + BC_RSTEP * i;
        const float ws = __builtin_amdgcn_exp2f((cse - sCS[s]) * kLog2eF) * sDL[s];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = ws * bf16_value(static_cast<unsigned short>(gb[i][e / 2] >> (16 * (e % 2))));
          const unsigned short hi = bf16_bits_of(v);
          sB[(bcc + e) * SQ + s] = hi;
          sWl[(bcc + e) * SQ + s] = bf16_bits_of(v - bf16_value(hi));
        }
      }
    }
    if (k + 1 < nchunks) load_b(t0 + Q);

    // ---- Y = exp(cs_t) C H_prev^T + M x  (wavefront w: token rows 16w..16w+15, 4 tiles of 16 channels)
    {
      f32x4_t yacc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) yacc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sC[(16 * w + lr) * SN + 32 * kk + 8 * lq]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&sHT[(16 * c + lr) * SN + 32 * kk + 8 * lq]);
          const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&sHl[(16 * c + lr) * SN + 32 * kk + 8 * lq]);
          yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, yacc[c], 0, 0, 0);
          yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, yacc[c], 0, 0, 0);
        }
      }
      const f32x4_t cst = *reinterpret_cast<const f32x4_t*>(&sCS[16 * w + 4 * lq]);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) yacc[c][j] *= __builtin_amdgcn_exp2f(cst[j] * kLog2eF);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (32 * kk > 16 * w + 15) continue;  // M is zero past the diagonal
        const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&sM[(16 * w + lr) * SQ + 32 * kk + 8 * lq]);
        const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&sMl[(16 * w + lr) * SQ + 32 * kk + 8 * lq]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&sXT[(16 * c + lr) * SQ + 32 * kk + 8 * lq]);
          yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb, yacc[c], 0, 0, 0);
          yacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb, yacc[c], 0, 0, 0);
        }
      }
      // epilogue: + D x, times SiLU(z), rounded to bf16
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int pch = 16 * c + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * w + 4 * lq + j;
          const int off = static_cast<int>(((t0 + t) * rowe + pch) * 2);
          float v = __builtin_fmaf(Dh, bf16_value(sXT[pch * SQ + t]), yacc[c][j]);
          if (p.z) v *= silu_f(bf16_value(static_cast<unsigned short>(__builtin_amdgcn_raw_buffer_load_b16(rs_z, off, 0, 0))));
          __builtin_amdgcn_raw_buffer_store_b16(bf16_bits_of(v), rs_y, off, 0, 0);
        }
      }
    }
    __syncthreads();  // W is staged; every read of H_prev is done

    // ---- H^T = exp(cs_end) H^T + x^T W  (wavefront w: channels 16w..16w+15, NT tiles of 16 states)
    {
      const float fade = __builtin_amdgcn_exp2f(sCS[Q - 1] * kLog2eF);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) hacc[nt][j] *= fade;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sXT[(16 * w + lr) * SQ + 32 * kk + 8 * lq]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&sB[(16 * nt + lr) * SQ + 32 * kk + 8 * lq]);
          const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&sWl[(16 * nt + lr) * SQ + 32 * kk + 8 * lq]);
          hacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, hacc[nt], 0, 0, 0);
          hacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, hacc[nt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int idx = (16 * w + 4 * lq + j) * SN + 16 * nt + lr;
          const unsigned short hi = bf16_bits_of(hacc[nt][j]);
          sHT[idx] = hi;
          sHl[idx] = bf16_bits_of(hacc[nt][j] - bf16_value(hi));
        }
    }
    __syncthreads();  // H^T is staged; x^T and W are free for the next chunk
  }

  if (p.final_state) {
    float* fs = p.final_state + ((b * H + h) * P) * N;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) fs[(16 * w + 4 * lq + j) * N + 16 * nt + lr] = hacc[nt][j];
  }
}

}  // namespace ssm
