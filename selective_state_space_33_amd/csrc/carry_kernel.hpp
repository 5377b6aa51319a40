// carry_kernel.hpp -- composition of chunk pairs into carried-in states, for
// tiles cut into many chunks ("Mamba is attention all you really need, part
// 2", "The relay": combine the chunk pairs in order, pass the real states
// back).  Included by ssm_scan.hip only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// State entering each chunk of a split tile: carry_{c+1} = P_c * carry_c + S_c,
// carry_0 = the tile's initial state (zero when h0 is null; h0 is
// [batch][dim][N]), for every column (lane channel, state) of the tile; layout
// [n_split][Ks][64][Npad].  The Ks-1 pairs of a column are cut into RUNS
// runs: each thread composes one run of one column into a single pair, the
// runs' pairs are combined in order through LDS, and each thread walks its
// run again from the state entering it, writing the carries.  A workgroup
// holds RUNS runs of 256 / RUNS columns.  RUNS = 1 (short chains): one thread
// walks a whole column, with no second walk.
constexpr int kCarryRuns = 32;
template <int RUNS> struct CarryShape {
  static_assert(RUNS >= 1 && 256 % RUNS == 0, "runs");
  static constexpr int COLS = 256 / RUNS;
};
constexpr int kCarryCols = CarryShape<kCarryRuns>::COLS;

template <int RUNS = kCarryRuns>
__global__ void __launch_bounds__(256) carry_kernel(const float* __restrict__ P, const float* __restrict__ S,
                                                   float* __restrict__ carry, int64_t n_split, int Ks, int64_t Npad,
                                                   const float* __restrict__ h0, int64_t n_long, int64_t ntd,
                                                   int64_t dim, int64_t N) {
  constexpr int kCols = CarryShape<RUNS>::COLS;
  __shared__ float sP[RUNS > 1 ? RUNS : 1][kCols], sS[RUNS > 1 ? RUNS : 1][kCols];
  const int run = threadIdx.x / kCols;
  const int cl = threadIdx.x % kCols;
  const int64_t per_tile = 64 * Npad;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * kCols + cl;  // over n_split * per_tile
  const bool ok = col < n_split * per_tile;
  const int64_t st = ok ? col / per_tile : 0, r = col % per_tile;
  const int npairs = Ks - 1;
  const int len = (npairs + RUNS - 1) / RUNS;
  const int c0 = run * len;
  const int c1 = (c0 + len < npairs) ? c0 + len : npairs;
  auto at = [&](int cc) { return (st * Ks + cc) * per_tile + r; };
  // this run's pair: (a, b) composed over chunks c0 .. c1-1, in order
  float a = 1.0f, bb = 0.0f;
  if (RUNS > 1 && ok) {
#pragma unroll 8
    for (int cc = c0; cc < c1; ++cc) {
      const float pc = P[at(cc)];
      a *= pc;
      bb = __builtin_fmaf(pc, bb, S[at(cc)]);
    }
  }
  if constexpr (RUNS > 1) {
    sP[run][cl] = a;
    sS[run][cl] = bb;
    __syncthreads();
  }
  // state entering this run: the tile's initial state, then the runs before it, composed in order
  float h = 0.0f;
  if (h0 && ok) {
    const int64_t tile = n_long + st;
    const int64_t d = (tile % ntd) * 64 + r / Npad, n = r % Npad;
    if (d < dim && n < N) h = h0[((tile / ntd) * dim + d) * N + n];
  }
  if constexpr (RUNS > 1)
    for (int q = 0; q < run; ++q) h = __builtin_fmaf(sP[q][cl], h, sS[q][cl]);
  if (!ok) return;
#pragma unroll 8
  for (int cc = c0; cc < c1; ++cc) {
    h = __builtin_fmaf(P[at(cc)], h, S[at(cc)]);
    carry[at(cc + 1)] = h;
  }
}

}  // namespace ssm
