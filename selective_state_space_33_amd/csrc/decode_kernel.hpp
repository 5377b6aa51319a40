// decode_kernel.hpp -- one-token recurrent step (decode) for gfx950.
//
// The state [batch, dim, dstate] is read and written exactly once, so the step
// is bound by HBM traffic on the state.  A group of NQ lanes owns one (b, d)
// channel and each lane four consecutive states, so a wavefront reads and
// writes the state as contiguous 16-byte-per-lane runs.  The partial readouts
// of the group are summed with cross-lane shuffles.  The per-channel
// prologue (softplus) is repeated by the NQ lanes of a group; it is a few
// instructions next to the state traffic.
#pragma once

#include "common.hpp"

namespace ssm {

struct DecodeParams {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;     // nullable
  const void* z;      // nullable
  const float* bias;  // nullable
  void* y;
  int64_t batch, dim, N;
  int softplus;
};

// NQ lanes per channel (power of two, 4 * NQ >= N); VEC4: dstate % 4 == 0.
template <class IO, int NQ, bool VEC4>
__global__ void __launch_bounds__(256) state_update_kernel(DecodeParams p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int q = static_cast<int>(gid & (NQ - 1));
  const int64_t bd = gid / NQ;
  const int64_t total = p.batch * p.dim;
  const bool valid = bd < total;
  const int64_t b = valid ? bd / p.dim : 0;
  const int64_t d = valid ? bd % p.dim : 0;
  const int64_t N = p.N;
  const int n0 = 4 * q;

  float h[4], A2[4], Bv[4], Cv[4];
  bool nok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) nok[j] = valid && (n0 + j) < N;
  if (VEC4 && nok[0]) {
    const float4 hv = *reinterpret_cast<const float4*>(p.state + bd * N + n0);
    const float4 av = *reinterpret_cast<const float4*>(p.A + d * N + n0);
    h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
    A2[0] = av.x * kLog2e; A2[1] = av.y * kLog2e; A2[2] = av.z * kLog2e; A2[3] = av.w * kLog2e;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = nok[j] ? p.state[bd * N + n0 + j] : 0.0f;
      A2[j] = nok[j] ? p.A[d * N + n0 + j] * kLog2e : 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    Bv[j] = nok[j] ? load_elem<IO>(p.B, b * N + n0 + j) : 0.0f;
    Cv[j] = nok[j] ? load_elem<IO>(p.C, b * N + n0 + j) : 0.0f;
  }
  const float uu = valid ? load_elem<IO>(p.u, bd) : 0.0f;
  const float x = (valid ? load_elem<IO>(p.delta, bd) : 0.0f) + ((valid && p.bias) ? p.bias[d] : 0.0f);
  const float dl = p.softplus ? softplus_f(x) : x;
  const float du = dl * uu;

  float yp = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = __builtin_amdgcn_exp2f(dl * A2[j]);
    h[j] = __builtin_fmaf(a, h[j], du * Bv[j]);
    yp = __builtin_fmaf(Cv[j], h[j], yp);
  }
  if (VEC4 && nok[0]) {
    *reinterpret_cast<float4*>(p.state + bd * N + n0) = make_float4(h[0], h[1], h[2], h[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (nok[j]) p.state[bd * N + n0 + j] = h[j];
  }
#pragma unroll
  for (int off = 1; off < NQ; off <<= 1) yp += __shfl_xor(yp, off, NQ);
  if (valid && q == 0) {
    float v = __builtin_fmaf(p.D ? p.D[d] : 0.0f, uu, yp);
    if (p.z) v *= silu_f(load_elem<IO>(p.z, bd));
    if constexpr (__is_same(IO, F32)) {
      static_cast<float*>(p.y)[bd] = v;
    } else {
      static_cast<uint16_t*>(p.y)[bd] = to_bf16(v);
    }
  }
}

// Vector path (dstate % 4 == 0, 16-byte aligned state and A, B/C rows aligned
// to 4 elements).  A thread owns one (channel d, group of 4 states) for R
// batch rows: A, bias and D are read once and reused, the R state quads are
// all in flight before any is used, and B_b/C_b come in as one 4-element
// vector load each.  Consecutive threads take consecutive state quads, so a
// wavefront reads and writes 1 KB of contiguous state per batch row.
template <class IO> struct Vec4In;
template <> struct Vec4In<F32> {
  static __device__ __forceinline__ void load(const void* base, int64_t idx, float* o) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct Vec4In<BF16> {
  static __device__ __forceinline__ void load(const void* base, int64_t idx, float* o) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
  }
};

// Sum of v over each aligned group of NQ lanes, left in every lane of the
// group: DPP quad permutations (lane i ^ 1, then i ^ 2) and, for eight lanes,
// the half-row mirror (lane i with 7 - i, which after the quad sums holds the
// other quad's sum); wider groups use cross-lane shuffles.
template <int NQ> __device__ __forceinline__ float group_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                              0xf, 0xf, false));
  };
  if constexpr (NQ >= 2) v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm(1, 0, 3, 2)
  if constexpr (NQ >= 4) v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm(2, 3, 0, 1)
  if constexpr (NQ >= 8) v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
#pragma unroll
  for (int off = 8; off < NQ; off <<= 1) v += __shfl_xor(v, off, NQ);
  return v;
}

template <class IO, int NQ, int R>
__global__ void __launch_bounds__(256) state_update_vec_kernel(DecodeParams p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int q = static_cast<int>(gid & (NQ - 1));
  const int64_t dq = gid / NQ;
  const int64_t dim = p.dim, N = p.N;
  const int64_t nbg = (p.batch + R - 1) / R;
  const bool valid = dq < dim * nbg;
  const int64_t d = valid ? dq % dim : 0;
  const int64_t b0 = valid ? (dq / dim) * R : 0;
  const int n0 = 4 * q;
  const bool qok = valid && n0 < N;
  const int64_t nc = qok ? n0 : 0;

  // Every load is issued up front and unconditionally, from an address clamped
  // into its array (a missing bias, D or z reads a same-sized array in its
  // place, and the value is then dropped); the invalid lanes' values are masked
  // after the loads.  Loads under divergent branches would each be waited for
  // before the next one issues: a memory round trip apiece.
  const float4 av = *reinterpret_cast<const float4*>(p.A + d * N + nc);
  const float bias_v = (p.bias ? p.bias : p.A)[d];
  const float D_v = (p.D ? p.D : p.A)[d];
  float h[R][4], Bv[R][4], Cv[R][4], uu[R], xr[R], zz[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t bc = (b0 + r < p.batch) ? b0 + r : p.batch - 1;
    const float4 hv = *reinterpret_cast<const float4*>(p.state + (bc * dim + d) * N + nc);
    h[r][0] = hv.x; h[r][1] = hv.y; h[r][2] = hv.z; h[r][3] = hv.w;
    Vec4In<IO>::load(p.B, bc * N + nc, Bv[r]);
    Vec4In<IO>::load(p.C, bc * N + nc, Cv[r]);
    uu[r] = load_elem<IO>(p.u, bc * dim + d);
    xr[r] = load_elem<IO>(p.delta, bc * dim + d);
    zz[r] = load_elem<IO>(p.z ? p.z : p.u, bc * dim + d);
  }
  const float A2[4] = {av.x * kLog2e, av.y * kLog2e, av.z * kLog2e, av.w * kLog2e};
  const float bias = p.bias ? bias_v : 0.0f;
  const float Dd = p.D ? D_v : 0.0f;

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t b = b0 + r;
    const bool ok = qok && b < p.batch;
    const float x = xr[r] + bias;
    float dl = softplus_f(x);
    dl = p.softplus ? dl : x;
    const float du = dl * uu[r];
    float yp = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = __builtin_amdgcn_exp2f(dl * A2[j]);
      h[r][j] = __builtin_fmaf(a, h[r][j], du * Bv[r][j]);
      yp = __builtin_fmaf(Cv[r][j], h[r][j], yp);
    }
    if (ok)
      *reinterpret_cast<float4*>(p.state + (b * dim + d) * N + n0) = make_float4(h[r][0], h[r][1], h[r][2], h[r][3]);
    yp = group_sum<NQ>(qok ? yp : 0.0f);  // quads past N read a clamped quad: they add nothing
    if (valid && b < p.batch && q == 0) {
      float v = __builtin_fmaf(Dd, uu[r], yp);
      if (p.z) v *= silu_f(zz[r]);
      if constexpr (__is_same(IO, F32)) {
        static_cast<float*>(p.y)[b * dim + d] = v;
      } else {
        static_cast<uint16_t*>(p.y)[b * dim + d] = to_bf16(v);
      }
    }
  }
}

}  // namespace ssm
