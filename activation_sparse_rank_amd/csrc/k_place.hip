// Neuron placement by profiled hotness.
//
// [QB] "Локальность вывода, вызванная редкой активацией": neuron firing
// follows a power law; a small share of neurons carries most activations.
// [QB] "Гибридный дизайн вывода CPU/GPU": before serving, each neuron's hot or
// cold character is analysed offline and decides where the neuron is placed.
// On one GPU every neuron stays in device memory, so placement here is a
// neuron's row position inside its layer: hot neurons are dealt evenly over
// the fused layer kernel's neuron segments (one workgroup each), which evens
// out the active rows per workgroup and so the number of dependent load
// rounds of the slowest one.  Renaming the neurons of a layer consistently in
// every per-neuron array leaves the layer's function unchanged.
//
//   k_count_active -- counts[i] += number of tokens t with mask[t][i] != 0
//   k_permute_rows -- dst row k = src row perm[k]
//   hot_order      -- (host) the placement order from the counts
#include <algorithm>
#include <numeric>
#include <vector>

#include "pi_internal.h"

namespace pi {
namespace {

constexpr int kPlThreads = 256;

__global__ __launch_bounds__(kPlThreads) void k_count_active(const uint8_t* __restrict__ mask, int n_tok, int d_ff,
                                                             uint32_t* __restrict__ counts) {
  const int i = blockIdx.x * kPlThreads + threadIdx.x;
  if (i >= d_ff) return;
  uint32_t c = 0;
  for (int t = 0; t < n_tok; ++t) c += mask[(size_t)t * d_ff + i] != 0 ? 1u : 0u;
  counts[i] += c;
}

// One workgroup per destination row; V16: 16-byte units (row_bytes % 16 == 0
// and both bases 16-byte aligned), else 4-byte units.
template <bool V16>
__global__ __launch_bounds__(kPlThreads) void k_permute_rows(const char* __restrict__ src, int rows, int row_bytes,
                                                             const int32_t* __restrict__ perm,
                                                             char* __restrict__ dst) {
  const int k = blockIdx.x;
  const int from = perm[k];
  const bool ok = (unsigned)from < (unsigned)rows;     // an entry outside [0, rows) gives a zero row
  const char* s = src + (size_t)(ok ? from : 0) * row_bytes;
  char* o = dst + (size_t)k * row_bytes;
  if (V16) {
    const int n = row_bytes / 16;
    for (int u = threadIdx.x; u < n; u += kPlThreads)
      reinterpret_cast<u32x4*>(o)[u] = ok ? reinterpret_cast<const u32x4*>(s)[u] : u32x4{0, 0, 0, 0};
  } else {
    const int n = row_bytes / 4;
    for (int u = threadIdx.x; u < n; u += kPlThreads)
      reinterpret_cast<uint32_t*>(o)[u] = ok ? reinterpret_cast<const uint32_t*>(s)[u] : 0u;
  }
}

}  // namespace

hipError_t launch_count_active(const uint8_t* mask, int n_tok, int d_ff, uint32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(k_count_active, dim3((d_ff + kPlThreads - 1) / kPlThreads), dim3(kPlThreads), 0, s, mask, n_tok,
                     d_ff, counts);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const void* src, int rows, int row_bytes, const int32_t* perm, void* dst,
                               hipStream_t s) {
  const bool v16 = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  const char* sb = static_cast<const char*>(src);
  char* db = static_cast<char*>(dst);
  if (v16)
    hipLaunchKernelGGL((k_permute_rows<true>), dim3(rows), dim3(kPlThreads), 0, s, sb, rows, row_bytes, perm, db);
  else
    hipLaunchKernelGGL((k_permute_rows<false>), dim3(rows), dim3(kPlThreads), 0, s, sb, rows, row_bytes, perm, db);
  return hipGetLastError();
}

// Neurons in order of decreasing count (ties: lower neuron first) are dealt
// over n_seg = ceil(d_ff / seg) segments of seg consecutive rows: the k-th
// neuron of that order takes slot k / n_seg of segment k % n_seg, the
// segments walked forward on even slots and backward on odd ones, so every
// segment receives one neuron of each band of n_seg ranks and the bands'
// leftovers alternate ends.  Positions past d_ff (a short last segment) are
// skipped.
void hot_order(const uint32_t* counts, int d_ff, int seg, int32_t* perm) {
  std::vector<int32_t> by(d_ff);
  std::iota(by.begin(), by.end(), 0);
  std::stable_sort(by.begin(), by.end(), [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
  const int n_seg = (d_ff + seg - 1) / seg;
  int k = 0;
  for (int q = 0; q < seg; ++q)
    for (int j = 0; j < n_seg; ++j) {
      const int sg = q % 2 == 0 ? j : n_seg - 1 - j;
      const long long pos = (long long)sg * seg + q;
      if (pos < d_ff) perm[pos] = by[k++];
    }
}

}  // namespace pi
