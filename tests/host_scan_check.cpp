// Host harness for the round tails' LDS scans (scan_best_lds, scan_top_lds): runs their index
// arithmetic on the CPU, for every simulated thread of a workgroup, over a stream held in a heap
// array of exactly the length the kernels guarantee readable (ids up to the next multiple of
// four past len - 1).  Built with AddressSanitizer, so any read below or past that array (the
// kind of read that faulted the tree drafter's LDS scan on the GPU) stops the run.
//
// stdin:  cases, then per case: len nmax nthreads, then len ids
// stdout: per case: l e (best of scan_best_lds; 0 0 when nothing matched), then the four best
//         keys of scan_top_lds merged over the threads, as l e pairs (0 0 past the last)
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../weight_bound_verify_amd/csrc/sv_tail.h"

int main() {
    int cases = 0;
    if (std::scanf("%d", &cases) != 1) return 2;
    for (int c = 0; c < cases; ++c) {
        int len = 0, nmax = 0, nthreads = 0;
        if (std::scanf("%d %d %d", &len, &nmax, &nthreads) != 3) return 2;
        std::vector<int32_t> ids(len);
        for (int i = 0; i < len; ++i)
            if (std::scanf("%d", &ids[i]) != 1) return 2;
        // readable extent: groups cover end positions 0 .. len-2, four per group
        const int ngroups = (len - 1 + 3) >> 2;
        const int extent = ngroups > 0 ? 4 * ngroups : 0;
        const size_t bytes = (size_t)(extent > len ? extent : len) * 4;
        int32_t* tk = static_cast<int32_t*>(std::aligned_alloc(16, bytes > 0 ? (bytes + 15) / 16 * 16 : 16));
        if (!tk) return 3;
        if (len > 0) std::memcpy(tk, ids.data(), (size_t)len * 4);
        // ids past the stream repeat its last id: a scan that compared them would find matches
        for (int i = len; i < (int)(bytes / 4); ++i) tk[i] = len > 0 ? ids[len - 1] : 0;
        int32_t suf[SV_MAX_NGRAM];
        for (int i = 0; i < SV_MAX_NGRAM; ++i) suf[i] = (i < nmax && len - 1 - i >= 0) ? tk[len - 1 - i] : -1;
        unsigned long long best = 0;
        std::vector<unsigned long long> keys;
        for (int t = 0; t < nthreads; ++t) {
            const unsigned long long b = nmax <= 4 ? sv::scan_best_lds<4>(tk, len, nmax, suf, t, nthreads)
                                                   : sv::scan_best_lds<8>(tk, len, nmax, suf, t, nthreads);
            best = b > best ? b : best;
            unsigned long long top[sv::kMaxBranches] = {0ull, 0ull, 0ull, 0ull};
            if (nmax <= 4) sv::scan_top_lds<4>(tk, len, nmax, suf, top, t, nthreads);
            else sv::scan_top_lds<8>(tk, len, nmax, suf, top, t, nthreads);
            for (unsigned long long k : top)
                if (k) keys.push_back(k);
        }
        std::sort(keys.begin(), keys.end(), [](unsigned long long a, unsigned long long b) { return a > b; });
        keys.resize(sv::kMaxBranches, 0ull);
        std::printf("%llu %llu", best >> 32, best & 0xffffffffull);
        for (unsigned long long k : keys) std::printf(" %llu %llu", k >> 32, k & 0xffffffffull);
        std::printf("\n");
        std::free(tk);
    }
    return 0;
}
