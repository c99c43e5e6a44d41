// Host-side shape rules of the kernels: which kernel a shape can take, how a
// launch is sized, how much LDS or scratch it needs.  Plain C++ (no device
// code), shared by the launchers and by the argument validation of api.cpp.
#include <algorithm>

#include "internal.h"

namespace bl {

// Workgroups per row of the split quantiser: enough to put about 256
// workgroups on the chip when the rows are few, each keeping at least 32
// chunks (512 elements) of its own; 1 (the one-workgroup-per-row kernel) from
// 5 rows up or for short rows.  Back-to-back times at K = 8192 (the launch
// alone is 3.2 us): one token 5.35 -> 5.07 us split 16 ways; 8 tokens 4.18 us
// in 8 workgroups against 4.34 split; 64 tokens 4.19 against 5.44 split 4 ways
// (each workgroup reads the whole row: the re-reads then cost more than the
// parallelism gains).
int quant_split_ways(int64_t M, int64_t K) {
    if (M <= 0 || M > 4) return 1;
    const int64_t by_rows = 256 / M;
    const int64_t by_len = (K / 16) / 32;
    return (int)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(by_rows, by_len), 64));
}

bool quant_gemv_supports(int M, int K, int N) {
    return M == 1 && K > 0 && K % 64 == 0 && K <= kFusedMaxK && N > 0 && N <= kFusedMaxN;
}

// LDS bytes of the decode kernel: the activation block rounded up to whole
// 1 KB copies, the reduction buffer, and 16 activation sums and 16 output
// scales per group.
int decode_a_bytes(int M, int K) { return ((M * K + 1023) / 1024) * 1024; }
size_t decode_lds_bytes(int M, int K, int ntw, int G) {
    return (size_t)decode_a_bytes(M, K) + (size_t)kDecWaves * ntw * 4 * 64 * 4 + 2 * 16 * 4 * (size_t)G;
}

// K parts of the decode widths, widest first: <8,2> 2, <4,2> 4, <2,1> 4, <1,1> 8.
// Grouped launches need KS % G == 0 and (K/256) % KS == 0 so that every wave's
// K range lies inside one group.
int grouped_width(int tiles, int G, int nchunks) {
    const int ct[4] = {8, 4, 2, 1}, ks[4] = {2, 4, 4, 8}, min_tiles[4] = {8 * 200, 4 * 200, 2 * 200, 0};
    int pick = -1;
    for (int i = 3; i >= 0; --i)  // the widest fitting config that still leaves >= 200 workgroups
        if (ks[i] % G == 0 && nchunks % ks[i] == 0 && (pick < 0 || tiles >= min_tiles[i])) pick = i;
    return pick < 0 ? -1 : ct[pick];
}

bool decode_lds_supports(int M, int K, int N) {
    return M >= 1 && M <= 16 && K >= 256 && K % 256 == 0 && N > 0 &&
           decode_lds_bytes(M, K, 2, 1) <= (size_t)kDecLdsMax;
}

// One token on the decode kernel (two K parts per tile) rather than the VALU
// GEMV: long rows over many row tiles.  Back-to-back times, bit-identical:
// K = 8192, N = 28672 12.9 -> 11.4 us (1-bit weights 11.0 -> 8.9 us); K = 4096,
// N = 11008 5.1 -> 4.8 us (1-bit 4.7 -> 4.5 us); at K = 2560, N = 6912 and
// K = N = 2048 the two are equal or the GEMV is faster.  The two-part unit is
// 512 inputs of 2-bit or 1024 of 1-bit weights.
bool decode_one_token(int K, int N, bool onebit) {
    return K >= 4096 && K % (onebit ? 1024 : 512) == 0 && N / 64 >= 150 &&
           decode_lds_supports(1, K, N);
}

bool decode_lds_grouped_supports(int M, int K, int G, int N) {
    if ((G != 2 && G != 4 && G != 8) || M < 1 || M > 16 || N <= 0 || K % 256 != 0 || K % G != 0 ||
        (K / G) % 256 != 0)
        return false;
    return grouped_width((N + 15) / 16, G, K >> 8) > 0 &&
           decode_lds_bytes(M, K, 2, G) <= (size_t)kDecLdsMax;
}

// Scratch of the pairwise float64 mean: one partial sum per leaf group of
// `group` entries, plus one level of sums of 64 of those when there are more
// than 64.
size_t pairwise_scratch_bytes(int64_t L, int group) {
    const int64_t n = (L + group - 1) / group;
    return (size_t)8 * (size_t)(n + (n > 64 ? (n + 63) / 64 : 0));
}

}  // namespace bl
