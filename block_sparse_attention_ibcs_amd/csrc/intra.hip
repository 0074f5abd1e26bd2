// INTRA relay patterns as kept-sub-block lists for the gather attention kernel.
//
// INTRA page (paperdot search page, query "Wenbo Lu"; abstract): static sparse
// patterns over computational query sets, built from complementary groups under a
// partition model. Scatter forms relay groups drawing on every local neighbourhood;
// Gather reconnects them. Readings: the computational query set is the query block;
// the sequence is cut into neighbourhoods of L tokens (L a multiple of q_block);
// Scatter keeps, in every neighbourhood, the keys at the offsets the query block
// covers in its own; Gather keeps the query block's own neighbourhood. Weight 1 for
// every kept sub-block, ascending lists.
//
// One workgroup per (b, h, query block). Entry e of a Gather row is sub-block
// j0 + e of the neighbourhood's run; with Bk <= Bq, entry e of a Scatter row is
// sub-block t of neighbourhood n (n = e / (Bq/Bk), t = e % (Bq/Bk)): every
// neighbourhood but the last contributes all Bq/Bk of its sub-blocks at the block's
// offset; with Bk > Bq each neighbourhood's slice is one sub-block.
#include "ab_internal.h"

namespace ab {
namespace {

__global__ __launch_bounds__(256) void intra_lists_kernel(Dims P, int layer, int L, int32_t* __restrict__ idx,
                                                          float* __restrict__ weights, int32_t* __restrict__ counts) {
  const int row = blockIdx.x;  // (b*H + h)*nqb + i
  const int i = row % P.nqb;
  const int N = P.N, Bq = P.Bq, Bk = P.Bk;
  const int p = (i * Bq) / L;     // neighbourhood of the query block
  const int o = i * Bq - p * L;   // its offset there (a multiple of Bq)
  int count;
  int j0 = 0;
  if (layer == AB_INTRA_GATHER) {
    j0 = (p * L) / Bk;
    const int end = min(N, (p + 1) * L);
    count = ceil_div(end, Bk) - j0;
  } else if (Bk > Bq) {
    // A slice of Bq tokens at a Bq-aligned offset lies inside one sub-block: one entry
    // per neighbourhood whose slice holds real tokens, each a different sub-block when
    // L >= Bk. L < Bk leaves L = Bq and offset 0, so consecutive slices pair up inside
    // one sub-block and together cover the sequence: every sub-block.
    const int ns = N > o ? ceil_div(N - o, L) : 0;
    count = L >= Bk ? ns : P.nkb;
  } else {
    // neighbourhoods whose slice at offset o holds real tokens, and the sub-blocks of
    // the last one (possibly cut by the end of the sequence)
    const int per = Bq / Bk;
    const int nfull = N / L + ((N % L) > o + Bq - 1 ? 1 : 0);  // slices entirely inside the sequence
    const bool part = (N % L) > o && (N % L) < o + Bq;         // one slice cut short by the end
    count = nfull * per + (part ? ceil_div(N % L - o, Bk) : 0);
    // (N / L counts the complete neighbourhoods; a partial last neighbourhood adds a
    // complete slice when it reaches past o + Bq, a cut one when it ends inside it)
  }
  int32_t* ri = idx + size_t(row) * P.nkb;
  float* rw = weights + size_t(row) * P.nkb;
  for (int e = threadIdx.x; e < count; e += blockDim.x) {
    int j;
    if (layer == AB_INTRA_GATHER) {
      j = j0 + e;
    } else if (Bk > Bq) {
      j = L >= Bk ? (e * L + o) / Bk : e;
    } else {
      const int per = Bq / Bk;
      const int n = e / per, t = e % per;
      j = (n * L + o) / Bk + t;
    }
    ri[e] = j;
    rw[e] = 1.0f;
  }
  if (threadIdx.x == 0) counts[row] = count;
}

// Processing order for the attention kernel: Scatter rows sharing an offset (hence
// one list) are placed next to each other, so the workgroups an XCD holds at once
// read the same keys; Gather keeps the natural order (its neighbourhoods are already
// contiguous). Position k of head bh's run: with U = L / q_block offsets and
// NQB = a U + r, offsets u < r have a + 1 query blocks and the rest a; the position
// runs over offsets, and within an offset over neighbourhoods.
__global__ __launch_bounds__(256) void intra_order_kernel(Dims P, int layer, int L, int32_t* __restrict__ order) {
  const int pos = blockIdx.x * blockDim.x + threadIdx.x;
  const int rows = P.B * P.H * P.nqb;
  if (pos >= rows) return;
  const int bh = pos / P.nqb, k = pos % P.nqb;
  int i = k;
  if (layer == AB_INTRA_SCATTER) {
    const int U = L / P.Bq;
    const int a = P.nqb / U, r = P.nqb % U;
    int u, p;
    if (k < r * (a + 1)) {
      u = k / (a + 1);
      p = k % (a + 1);
    } else {
      const int k2 = k - r * (a + 1);  // a > 0 here: positions past the first r runs exist only then
      u = r + k2 / a;
      p = k2 % a;
    }
    i = p * U + u;
  }
  order[pos] = bh * P.nqb + i;
}

}  // namespace

hipError_t launch_intra_lists(const Dims& P, int layer, int partition_tokens, int32_t* idx, float* weights,
                              int32_t* counts, int32_t* row_order, hipStream_t s) {
  const int rows = P.B * P.H * P.nqb;
  hipLaunchKernelGGL(intra_lists_kernel, dim3(rows), dim3(256), 0, s, P, layer, partition_tokens, idx, weights,
                     counts);
  if (row_order)
    hipLaunchKernelGGL(intra_order_kernel, dim3(ceil_div(rows, 256)), dim3(256), 0, s, P, layer, partition_tokens,
                       row_order);
  return hipGetLastError();
}

int intra_default_partition(const Dims& P) {
  int r = 1;
  while (r * r < P.nqb) ++r;  // ceil(sqrt(NQB))
  return P.Bq * r;
}

}  // namespace ab
