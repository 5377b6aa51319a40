// order_kernel.hpp -- longest-first launch order of packed sequences.
//
// Each (tile column, sequence) unit of a packed scan runs its sequence start
// to end, so a unit's time grows with its length.  Workgroups start in index
// order as CUs free up; units handed out longest first keep the last ones
// short, which bounds the idle tail (longest-processing-time-first list
// scheduling).  The offsets live on the device, so one workgroup bins the
// sequences by length (1024 bins over [0, longest]) and writes the order,
// longest bin first.  Within a bin the order is whatever the LDS atomics give:
// every unit's outputs are its own, so the order changes no result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr int kOrderBins = 1024;

// order[0 .. nseq) = a permutation of the sequences 0 .. nseq-1, longest
// (offsets clamped into [0, L] as the scan clamps them) first.
static __global__ __launch_bounds__(kOrderBins) void packed_order_kernel(const int64_t* __restrict__ cu, int nseq,
                                                                  int64_t L, int* __restrict__ order) {
  __shared__ int bins[kOrderBins];
  __shared__ int longest;
  const int t = threadIdx.x;
  auto len_of = [&](int c) -> int {
    int64_t a = cu[c];
    a = a < 0 ? 0 : (a > L ? L : a);
    int64_t e = cu[c + 1];
    e = e < a ? a : (e > L ? L : e);
    return static_cast<int>(e - a);
  };
  bins[t] = 0;
  if (t == 0) longest = 0;
  __syncthreads();
  int m = 0;
  for (int c = t; c < nseq; c += kOrderBins) m = max(m, len_of(c));
  atomicMax(&longest, m);
  __syncthreads();
  const int64_t top = static_cast<int64_t>(longest) + 1;
  // bin 0 holds the longest sequences
  auto bin_of = [&](int len) {
    return kOrderBins - 1 - static_cast<int>(static_cast<int64_t>(len) * kOrderBins / top);
  };
  for (int c = t; c < nseq; c += kOrderBins) atomicAdd(&bins[bin_of(len_of(c))], 1);
  __syncthreads();
  // exclusive prefix sum of the bin counts: each bin's first slot
  const int own = bins[t];
  for (int o = 1; o < kOrderBins; o <<= 1) {
    const int add = t >= o ? bins[t - o] : 0;
    __syncthreads();
    bins[t] += add;
    __syncthreads();
  }
  bins[t] -= own;
  __syncthreads();
  for (int c = t; c < nseq; c += kOrderBins) order[atomicAdd(&bins[bin_of(len_of(c))], 1)] = c;
}

}  // namespace ssm
