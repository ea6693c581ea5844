// Standalone vocab-wide row statistics: one workgroup per (row, chunk); the workgroup
// that completes a row last merges its chunks (max, argmax, log-sum-exp, top-K).
#include "dtv_internal.h"
#include "rowstats.h"

namespace dtv {

constexpr int kRowStatsMaxK = 1024;
constexpr int kRowStatsMergeCap = 8192;  // chunks_of(V) * K must not exceed this

template <int DT>
__global__ __launch_bounds__(kBlock) void row_stats_kernel(RowStatsArgs a) {
  __shared__ RowSmem sm;
  __shared__ unsigned long long sortbuf[pow2_at_least(kWaves * kRowStatsMaxK)];
  row_smem_init(sm);
  __syncthreads();
  __shared__ MergeSmem<kRowStatsMergeCap> ms;
  using Rw = RowT<DT>;
  const int r = blockIdx.x / a.nch;
  const int c = blockIdx.x % a.nch;
  const int src = a.row_idx ? a.row_idx[r] : r;
  const char* row = static_cast<const char*>(a.table) + static_cast<size_t>(src) * a.V * Rw::ESIZE;
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
  const size_t ci = static_cast<size_t>(r) * a.nch + c;
  const int K = a.K;
  chunk_reduce<DT>(x, key, c, a.V, K, &a.st[ci], a.cval + ci * K, a.cidx + ci * K, sortbuf, sm);
  if (last_arrival(&a.tickets[r], a.nch, &sm.flag)) {
    const size_t rb = static_cast<size_t>(r) * a.nch;
    row_merge(a.st + rb, a.cval + rb * K, a.cidx + rb * K, a.nch, K,
              a.maxv ? a.maxv + r : nullptr, a.argmax ? a.argmax + r : nullptr,
              a.lse ? a.lse + r : nullptr, a.mval + static_cast<size_t>(r) * K,
              a.topk ? a.topk + static_cast<size_t>(r) * K : nullptr, sm, ms);
  }
}

int launch_row_stats(const RowStatsArgs& a, int dtype, hipStream_t st) {
  const dim3 grid(a.R * a.nch);
  if (dtype == 1)
    DTV_LAUNCH(row_stats_kernel<1>, grid, dim3(kBlock), 0, st, a);
  else
    DTV_LAUNCH(row_stats_kernel<0>, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
