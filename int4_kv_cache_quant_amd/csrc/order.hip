// order.hip - the order in which the split blocks of a batch take their
// work items.
//
// A batch of sequences of unequal length (a ragged batch) gives the split
// pass items of unequal size: full chunks, the sequences' last partial
// chunks, and empty ones.  The hardware starts workgroups in index order as
// compute units free up, so handing the items out longest first (the full
// chunks, then the partial ones by decreasing length, then the empty ones,
// which leave at once) is a longest-processing-time-first schedule: the long
// items no longer pile up on a few compute units at the end.  This kernel
// writes, for every block of the split grid, which item it takes; which
// block computes a partial does not change the partial, so the combine is
// unaffected.  Items only depend on lens[], which is on the device, hence a
// kernel rather than host code.
#include "common.hpp"
#include "kernels.hpp"

namespace otq {

namespace {

constexpr int kThreads = 256;

// One workgroup.  Per sequence b: nf full chunks and a last chunk of rem
// tokens.  Item j < F (F = total full chunks) is full chunk j in sequence
// order; item F + r is the last chunk of rank r (decreasing rem, then
// increasing b) among the sequences with rem > 0; the others are empty.
// Block k takes item k / groups with KV-head group k % groups.
__global__ __launch_bounds__(kThreads) void split_order_kernel(const int32_t* __restrict__ lens, int lens_offset,
                                                               int max_len, int chunk, int S, int groups,
                                                               int B, int2* __restrict__ items,
                                                               unsigned* __restrict__ err)
{
    __shared__ int nf[kOrderMaxBatch], rem[kOrderMaxBatch], pf[kOrderMaxBatch + 1];
    __shared__ int by_rank[kOrderMaxBatch];
    const int t = threadIdx.x;
    for (int b = t; b < B; b += kThreads) {
        const int raw = lens[b];
        if (raw < 0 || raw > max_len) report_error(err, kErrLens);
        const int len = max(min(max(raw, 0), max_len) - lens_offset, 0);  // as the split kernels
        nf[b] = len / chunk;
        rem[b] = len - nf[b] * chunk;
    }
    __syncthreads();
    if (t == 0) {  // exclusive prefix sums of nf (B <= 256: a short serial loop)
        int acc = 0;
        for (int b = 0; b < B; ++b) {
            pf[b] = acc;
            acc += nf[b];
        }
        pf[B] = acc;
    }
    for (int b = t; b < B; b += kThreads) {
        if (rem[b] > 0) {
            int rank = 0;
            for (int o = 0; o < B; ++o) rank += (rem[o] > rem[b] || (rem[o] == rem[b] && o < b)) ? 1 : 0;
            by_rank[rank] = b;
        }
    }
    __syncthreads();
    const int F = pf[B];
    int npart = 0;
    for (int b = 0; b < B; ++b) npart += rem[b] > 0 ? 1 : 0;
    const int n = S * groups * B;
    for (int k = t; k < n; k += kThreads) {
        const int j = k / groups;
        int2 it = make_int2(-1, 0);
        if (j < F) {
            int lo = 0, hi = B - 1;  // the last sequence whose chunks start at or before item j
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (pf[mid] <= j) lo = mid; else hi = mid - 1;
            }
            // (the last such sequence has full chunks: j < F)
            it = make_int2(j - pf[lo], lo);
        } else if (j - F < npart) {
            const int b = by_rank[j - F];
            it = make_int2(nf[b], b);
        }
        items[k] = it;
    }
}

}  // namespace

hipError_t launch_split_order(const int32_t* lens, int lens_offset, int max_len, int chunk, int S,
                              int groups, int B, int2* items, unsigned* err, hipStream_t stream)
{
    if (B < 2 || B > kOrderMaxBatch || chunk <= 0) return hipErrorInvalidValue;
    split_order_kernel<<<1, kThreads, 0, stream>>>(lens, lens_offset, max_len, chunk, S, groups, B, items, err);
    return hipGetLastError();
}

}  // namespace otq
