// scan_kernels.hpp -- gfx950 kernels of the selective scan forward pass.
//
// Work decomposition.  A workgroup owns 64 consecutive channels d of one batch
// row and one chunk of the sequence.  It has G wavefronts; wavefront w owns
// the states n in [w*NPL, (w+1)*NPL) of those 64 channels, one channel per
// lane, so each lane runs NPL independent fp32 recurrences in registers and
// B_t, C_t for its states are wave-uniform (scalar loads).
//
// Per block of TB tokens the workgroup
//   1. (prologue, all threads) loads u, delta_raw, z for TB x 64 tokens x
//      channels with coalesced vector loads, computes delta = softplus(raw +
//      bias) and delta*u once per (token, channel) and stages them in LDS;
//   2. (scan, each wavefront) walks the TB tokens: for every state
//      a = exp2(delta * A*log2 e), h = a*h + (delta*u)*B_t[n], and the partial
//      readout y_w = sum over its states of C_t[n]*h -- the pair (a, b) of the
//      fade-and-add step never leaves registers;
//   3. (epilogue, all threads) sums the G partial readouts in a fixed order,
//      adds D*u, multiplies by SiLU(z), rounds and stores y.
// Loads of the next block are issued before the scan of the current one.
//
// Long sequences are cut into K chunks ("Mamba is attention all you really
// need, part 2", "The relay": squash each chunk into one fade-and-add pair,
// combine the chunk pairs, pass the real states back):
//   chunk_agg   (FULL = false) scans chunks 0..K-2 from a zero state and
//               writes each chunk's pair (P, S) per (b, d, n): S is the state
//               the chunk reaches from zero, P = exp(A * sum of its deltas)
//               its total fade;
//   carry       composes the pairs in order and writes the state entering
//               every chunk;
//   scan (FULL = true) rescans every chunk from its carried-in state and
//               produces y and the final state.
#pragma once

#include "common.hpp"

namespace ssm {

struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  void* y;
  float* final_state;  // nullable
  float* aggP;         // [batch][K][dim][N]  (K > 1 only)
  float* aggS;         // [batch][K][dim][N]
  float* carry;        // [batch][K][dim][N]  state entering chunk c (c >= 1)
  int64_t batch, L, dim, N;
  int64_t chunk_len;
  int K;
  int softplus;
};

// Tokens per staged block for a (G, VW) variant: 16 or G*VW, whichever is larger.
template <int G, int VW> struct BlockShape {
  static constexpr int TB = (G * VW > 16) ? G * VW : 16;
  static constexpr int RPT = TB / (G * VW);  // rows handled by each prologue thread
};

// B_t / C_t of this wavefront's states n0 .. n0+NPL-1 for one token row
// (flat offset rowoff = row * N).  EXACT (NPL * G == N): the states split
// evenly over the wavefronts and no masking is needed.  Otherwise states
// n >= N read a clamped, in-bounds element and are set to zero (their A is
// zero too, so they stay at zero and add nothing to the readout).
template <class IO, int NPL, bool EXACT>
__device__ __forceinline__ void load_bc(const void* base, int64_t rowoff, int n0, int64_t N, float* v) {
  if constexpr (EXACT) {
    Row<IO, NPL>::load(base, rowoff + n0, v);
  } else {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int64_t n = n0 + j;
      float x[1];
      Row<IO, 1>::load(base, rowoff + (n < N ? n : N - 1), x);
      v[j] = n < N ? x[0] : 0.0f;
    }
  }
}

// Tokens whose B/C words a wavefront preloads into SGPRs at once (about 32
// SGPRs for B and C together).
template <class IO, int NPL> struct Preload {
  static constexpr int WORDS = __is_same(IO, BF16) ? (NPL >= 2 ? NPL / 2 : 1) : NPL;  // dwords per token
  static constexpr int SUB = (16 / WORDS) > 0 ? 16 / WORDS : 1;
};

// NT: dstate as a compile-time constant when the states split evenly
// (NT = NPL * G), or 0 when it is only known at run time.
template <class IO, int NPL, int G, int VW, bool FULL, int NT>
__global__ void __launch_bounds__(64 * G) scan_kernel(ScanParams p) {
  constexpr bool EXACT = NT > 0;
  static_assert(NT == 0 || NT == NPL * G, "compile-time dstate must equal NPL * G");
  constexpr int TB = BlockShape<G, VW>::TB;
  constexpr int RPT = BlockShape<G, VW>::RPT;
  constexpr int RPR = 64 / VW;              // prologue threads per token row
  constexpr int ROWSTEP = (64 * G) / RPR;   // rows between one thread's runs
  static_assert(TB == RPT * ROWSTEP, "block shape");

  __shared__ float2 sDU[TB][64];                 // (delta, delta*u) per token, channel
  __shared__ float sY[FULL ? G : 1][TB][64];     // partial readouts per wavefront

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b = blockIdx.y;
  const int c = blockIdx.z;
  const int64_t dim = p.dim, L = p.L;
  const int64_t N = EXACT ? static_cast<int64_t>(NT) : p.N;
  const int64_t d0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t t_begin = static_cast<int64_t>(c) * p.chunk_len;
  const int64_t t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;

  // ---- scan lane: channel d, states n0 .. n0+NPL-1
  const int64_t d = d0 + lane;
  const bool dvalid = d < dim;
  const int n0 = w * NPL;
  float A2[NPL], h[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = n0 + j;
    const bool ok = dvalid && n < N;
    A2[j] = ok ? p.A[d * N + n] * kLog2e : 0.0f;
    h[j] = 0.0f;
    if (FULL && c > 0 && ok) h[j] = p.carry[((b * p.K + c) * dim + d) * N + n];
  }
  float delta_total = 0.0f;  // chunk sum of delta (aggregate pass), summed per block then per chunk

  // ---- prologue / epilogue thread: channels pd .. pd+VW-1, rows prow + i*ROWSTEP
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

  Raw<IO, VW> ru[RPT], rd[RPT], rz[RPT];  // loads for the block about to be staged
  Raw<IO, VW> eu[RPT], ez[RPT];           // u, z of the block awaiting its epilogue

  auto issue_loads = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int64_t t = t0 + prow + i * ROWSTEP;
      if (pvalid && t < t_end) {
        const int64_t idx = (b * L + t) * dim + pd;
        ru[i] = raw_load<IO, VW>(p.u, idx);
        rd[i] = raw_load<IO, VW>(p.delta, idx);
        rz[i] = has_z ? raw_load<IO, VW>(p.z, idx) : raw_zero<IO, VW>();
      } else {
        ru[i] = raw_zero<IO, VW>();
        rd[i] = raw_zero<IO, VW>();
        rz[i] = raw_zero<IO, VW>();
      }
    }
  };

  auto epilogue = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = prow + i * ROWSTEP;
      const int64_t t = t0 + row;
      if (!pvalid || t >= t_end) continue;
      float ys[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) ys[e] = 0.0f;
#pragma unroll
      for (int ww = 0; ww < G; ++ww) {
        if constexpr (VW == 4) {
          const float4 v = *reinterpret_cast<const float4*>(&sY[ww][row][pcol]);
          ys[0] += v.x; ys[1] += v.y; ys[2] += v.z; ys[3] += v.w;
        } else {
          ys[0] += sY[ww][row][pcol];
        }
      }
      float uf[VW], zf[VW], out[VW];
      unpack<IO, VW>(eu[i], uf);
      if (has_z) unpack<IO, VW>(ez[i], zf);
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        float v = __builtin_fmaf(Dv[e], uf[e], ys[e]);
        if (has_z) v *= silu_f(zf[e]);
        out[e] = v;
      }
      store_vals<IO, VW>(p.y, (b * L + t) * dim + pd, out);
    }
  };

  issue_loads(t_begin);
  int64_t t_prev = -1;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TB) {
    const int nt = static_cast<int>((t_end - t0 < TB) ? (t_end - t0) : TB);
    if (FULL && t_prev >= 0) epilogue(t_prev);

    // prologue: stage (delta, delta*u) for this block
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = prow + i * ROWSTEP;
      float uf[VW], df[VW];
      unpack<IO, VW>(ru[i], uf);
      unpack<IO, VW>(rd[i], df);
      float2 out[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const float x = df[e] + biasv[e];
        const float dl = p.softplus ? softplus_f(x) : x;
        out[e] = make_float2(dl, dl * uf[e]);
      }
      if constexpr (VW == 4) {
        float4* dst = reinterpret_cast<float4*>(&sDU[row][pcol]);
        dst[0] = make_float4(out[0].x, out[0].y, out[1].x, out[1].y);
        dst[1] = make_float4(out[2].x, out[2].y, out[3].x, out[3].y);
      } else {
        sDU[row][pcol] = out[0];
      }
      if (FULL) {
        eu[i] = ru[i];
        ez[i] = rz[i];
      }
    }
    issue_loads(t0 + TB);
    __syncthreads();

    // scan: TB tokens for this wavefront's states
    const int64_t row0 = b * L + t0;
    float block_delta = 0.0f;
    auto step = [&](int tt) {
      const float2 dd = sDU[tt][lane];
      const int64_t rowoff = (row0 + tt) * N;
      float Bv[NPL], Cv[NPL];
      load_bc<IO, NPL, EXACT>(p.B, rowoff, n0, N, Bv);
      if (FULL) load_bc<IO, NPL, EXACT>(p.C, rowoff, n0, N, Cv);
      float yp = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const float a = __builtin_amdgcn_exp2f(dd.x * A2[j]);
        h[j] = __builtin_fmaf(a, h[j], dd.y * Bv[j]);
        if (FULL) yp = __builtin_fmaf(Cv[j], h[j], yp);
      }
      if (FULL) sY[w][tt][lane] = yp;
      else block_delta += dd.x;
    };
    if (EXACT && nt == TB) {
      // Full block: issue the scalar loads of SUB tokens' B/C words back to back,
      // then run those tokens, so the scalar-load latency is paid once per SUB.
      constexpr int SUB = Preload<IO, NPL>::SUB;
      constexpr int WORDS = Preload<IO, NPL>::WORDS;
      static_assert(TB % SUB == 0, "sub-block");
      cu32_p Bp = (cu32_p)(p.B);
      cu32_p Cp = (cu32_p)(p.C);
      constexpr int ES = __is_same(IO, BF16) ? 2 : 1;   // elements per dword
#pragma unroll
      for (int s0 = 0; s0 < TB; s0 += SUB) {
        uint32_t bw[SUB][WORDS], cw[SUB][WORDS];
        const int64_t wbase = ((row0 + s0) * N + n0) / ES;   // dword index of token s0, state n0
#pragma unroll
        for (int q = 0; q < SUB; ++q) {
#pragma unroll
          for (int k = 0; k < WORDS; ++k) {
            bw[q][k] = Bp[wbase + (q * N) / ES + k];
            if (FULL) cw[q][k] = Cp[wbase + (q * N) / ES + k];
          }
        }
#pragma unroll
        for (int q = 0; q < SUB; ++q) {
          const int tt = s0 + q;
          const float2 dd = sDU[tt][lane];
          float Bv[NPL], Cv[NPL];
#pragma unroll
          for (int j = 0; j < NPL; ++j) {
            if constexpr (__is_same(IO, BF16)) {
              if constexpr (NPL == 1) {
                Bv[j] = (n0 & 1) ? bf16_hi(bw[q][0]) : bf16_lo(bw[q][0]);
                Cv[j] = FULL ? ((n0 & 1) ? bf16_hi(cw[q][0]) : bf16_lo(cw[q][0])) : 0.0f;
              } else {
                Bv[j] = (j & 1) ? bf16_hi(bw[q][j / 2]) : bf16_lo(bw[q][j / 2]);
                Cv[j] = FULL ? ((j & 1) ? bf16_hi(cw[q][j / 2]) : bf16_lo(cw[q][j / 2])) : 0.0f;
              }
            } else {
              Bv[j] = __uint_as_float(bw[q][j]);
              Cv[j] = FULL ? __uint_as_float(cw[q][j]) : 0.0f;
            }
          }
          float yp = 0.0f;
#pragma unroll
          for (int j = 0; j < NPL; ++j) {
            const float a = __builtin_amdgcn_exp2f(dd.x * A2[j]);
            h[j] = __builtin_fmaf(a, h[j], dd.y * Bv[j]);
            if (FULL) yp = __builtin_fmaf(Cv[j], h[j], yp);
          }
          if (FULL) sY[w][tt][lane] = yp;
          else block_delta += dd.x;
        }
      }
    } else {
      for (int tt = 0; tt < nt; ++tt) step(tt);
    }
    delta_total += block_delta;
    __syncthreads();
    t_prev = t0;
  }
  if (FULL && t_prev >= 0) epilogue(t_prev);

#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = n0 + j;
    if (!(dvalid && n < N)) continue;
    if (FULL) {
      if (c == p.K - 1 && p.final_state) p.final_state[(b * dim + d) * N + n] = h[j];
    } else {
      const int64_t idx = ((b * p.K + c) * dim + d) * N + n;
      p.aggS[idx] = h[j];
      p.aggP[idx] = __builtin_amdgcn_exp2f(A2[j] * delta_total);
    }
  }
}

// State entering each chunk: carry_{c+1} = P_c * carry_c + S_c, carry_0 = 0.
// One thread per (b, d, n); the chunk pairs are composed in order.
__global__ void __launch_bounds__(256) carry_kernel(const float* __restrict__ P, const float* __restrict__ S,
                                                   float* __restrict__ carry, int64_t batch, int K, int64_t DN) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= batch * DN) return;
  const int64_t b = i / DN, r = i % DN;
  float h = 0.0f;
  for (int cc = 0; cc + 1 < K; ++cc) {
    const int64_t idx = (b * K + cc) * DN + r;
    h = __builtin_fmaf(P[idx], h, S[idx]);
    carry[idx + DN] = h;
  }
}

}  // namespace ssm
