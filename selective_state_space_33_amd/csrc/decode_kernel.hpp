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

}  // namespace ssm
