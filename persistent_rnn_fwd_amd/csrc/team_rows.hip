// Sparse fp16 layers whose rows hold different numbers of nonzeros: the
// ordering kernel and the kernel instances (sparse_team_kernel, RAGGED).
//
// "Sparse Persistent RNNs: Squeezing Large Recurrent Networks On-Chip" (table
// "Measured effects reported in the paper", load-balanced pruning row) sets
// load-balanced pruning, equal nonzeros in every row, against plain pruning,
// whose rows differ in length.  Stored at the width of the longest row, such a
// layer costs every row the longest row's work.  Here each row's length is an
// input; the rows are ordered by how many 64-pair slots they fill (most
// first) and dealt to the waves in snake order by the kernel, so that each
// wave's rows have about the same slots in all; a wave runs its rows up to the
// slots of its longest row, not the layer's.
#include "team_kernel.h"

namespace prnn {

namespace {

constexpr int kSortThreads = 512;
constexpr int kSortKeys = kSparseRowsMaxK / 64 + 1;  // slot counts 0 .. 16

// Stable counting sort by slot count, one workgroup per segment of `seg`
// rows (the whole layer, or one XCD's part of it on two XCDs per batch row):
// workgroup g orders rows [g seg, min(n, (g + 1) seg)) and writes them, as
// layer row indexes, to the same range of `sorted`.  Thread t owns rows
// [t tseg, (t + 1) tseg) of the segment: it counts them per key into its own
// column of cnt, the columns are scanned in (key, thread) order, and each
// thread then writes its rows to their places in row order.  Key 0 = the
// most slots.
__global__ void __launch_bounds__(kSortThreads) sort_rows_kernel(const int32_t* row_len, int n, int k, int seg,
                                                                 int32_t* sorted) {
  __shared__ int cnt[kSortKeys * kSortThreads];  // [key][thread]
  __shared__ int part[kSortThreads];
  const int t = threadIdx.x;
  const int base = (int)blockIdx.x * seg;
  const int len = min(seg, n - base);
  const int tseg = (len + kSortThreads - 1) / kSortThreads;
  const int lo = min(len, t * tseg), hi = min(len, lo + tseg);
  auto key_of = [&](int r) {
    const int rl = min(max(row_len[base + r], 0), k);
    return (kSortKeys - 1) - ((rl + 63) >> 6);
  };
  for (int key = 0; key < kSortKeys; ++key) cnt[key * kSortThreads + t] = 0;
  for (int r = lo; r < hi; ++r) cnt[key_of(r) * kSortThreads + t] += 1;  // this thread's column only
  __syncthreads();
  // exclusive scan of cnt in memory order, kSortKeys consecutive entries per thread
  int local[kSortKeys], sum = 0;
#pragma unroll
  for (int i = 0; i < kSortKeys; ++i) {
    local[i] = cnt[t * kSortKeys + i];
    sum += local[i];
  }
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < kSortThreads; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
#pragma unroll
  for (int i = 0; i < kSortKeys; ++i) {
    cnt[t * kSortKeys + i] = run;
    run += local[i];
  }
  __syncthreads();
  for (int r = lo; r < hi; ++r) {
    const int c = key_of(r) * kSortThreads + t;
    sorted[base + cnt[c]] = base + r;
    cnt[c] += 1;
  }
}

}  // namespace

void launch_sort_rows(const int32_t* row_len, int n, int k, int seg, int32_t* sorted, hipStream_t stream) {
  hipLaunchKernelGGL(sort_rows_kernel, dim3((n + seg - 1) / seg), dim3(kSortThreads), 0, stream, row_len, n, k, seg,
                     sorted);
}

// (rows per wave, 64-pair slots of the longest row)
const KernelEntry kSparseRowsF16Kernels[] = {
    PRNN_SPARSE_ROWS(1, 1), PRNN_SPARSE_ROWS(2, 1), PRNN_SPARSE_ROWS(2, 2), PRNN_SPARSE_ROWS(4, 2),
    PRNN_SPARSE_ROWS(4, 4), PRNN_SPARSE_ROWS(7, 3), PRNN_SPARSE_ROWS(7, 5), PRNN_SPARSE_ROWS(8, 4),
    {0, 0, 0, nullptr},
};
// 12-wave workgroups: the 2304-neuron layers (6 rows per wave), rows of up to
// 256 and 640 pairs.
const KernelEntry kSparseRowsF16Kernels12[] = {
    PRNN_SPARSE_ROWS12(6, 4), PRNN_SPARSE_ROWS12(6, 10),
    {0, 0, 0, nullptr},
};

}  // namespace prnn
