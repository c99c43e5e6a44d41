// Output stage shared by the MFMA kernels: y = fl32(acc) * s_m with
// acc = D - S_m and s_m = fl32(beta * gamma_m) / 128 (unite.ai BitNet.cpp
// article, 3. BitLinear-Betrieb: output scaled by beta * gamma / Qb).
//
// A wave holds TM x TN accumulator tiles of 32 x 32 from
// v_mfma_i32_32x32x32_i8: lane l holds column l % 32 and, in register v, row
// 8 * (v / 4) + 4 * (l / 32) + v % 4 of each tile.  The per-row S_m and s_m
// come from block-local LDS arrays, so four consecutive rows are one 16-byte
// LDS read.
//
// y == nullptr stores only the accumulators (acc_out).
//
// Tiles wholly inside the output take a path without per-element bounds
// tests: one 32-bit row offset per row, column tiles addressed from
// wave-uniform base pointers, so each store is one instruction on an SGPR
// base.  Edge tiles test every element.
#pragma once

#include "device_common.h"

namespace bl {

typedef int v16i __attribute__((ext_vector_type(16)));

// Fill the block-local row tables: S[r] = sum of the `parts` partial sums
// Sp[p * rows + r], sc[r] = output scale of row m0 + r (0 past M).
// Called by every thread of the block between two barriers.
__device__ __forceinline__ void epilogue_tables(const int* Sp, int parts, int rows, int m0, int M,
                                                const float* gamma, float beta, int* S,
                                                float* sc, int tid, int nthreads) {
    for (int r = tid; r < rows; r += nthreads) {
        int s = 0;
        for (int p = 0; p < parts; ++p) s += Sp[p * rows + r];
        S[r] = s;
        const int row = m0 + r;
        sc[r] = (row < M) ? out_scale(beta, gamma[row]) : 0.f;
    }
}

// Store the wave's tiles.  (r0, c0): block-local first row / column of the
// wave's tile; (m0, n0): first row / column of the block tile.  S and sc are
// the block-local tables (16-byte aligned, r0 a multiple of 32).
template <int TM, int TN>
__device__ __forceinline__ void store_tiles(const v16i (&acc)[TM][TN], const int* S, const float* sc,
                                            int r0, int c0, int m0, int n0, int M, int N,
                                            float* __restrict__ y, int32_t* __restrict__ acc_out,
                                            int lane) {
    const int l32 = lane & 31, h = lane >> 5;
    const int row_w = m0 + r0, col_w = n0 + c0;
    const bool inside = row_w + TM * 32 <= M && col_w + TN * 32 <= N &&
                        (int64_t)TM * 32 * N < (int64_t)1 << 31;
    if (inside) {
        int32_t* aw = acc_out ? acc_out + (int64_t)row_w * N + col_w : nullptr;
        if (y) {
            float* yw = y + (int64_t)row_w * N + col_w;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int rb = 32 * i + 8 * g + 4 * h;  // wave-local row of v = 4g
                    const v4i s4 = *reinterpret_cast<const v4i*>(S + r0 + rb);
                    const v4f c4 = *reinterpret_cast<const v4f*>(sc + r0 + rb);
#pragma unroll
                    for (int vv = 0; vv < 4; ++vv) {
                        const uint32_t off = (uint32_t)(rb + vv) * (uint32_t)N + (uint32_t)l32;
#pragma unroll
                        for (int t = 0; t < TN; ++t) {
                            const int a = acc[i][t][4 * g + vv] - s4[vv];
                            float* yt = yw + 32 * t;
                            yt[off] = (float)a * c4[vv];
                        }
                    }
                }
            }
        }
        if (aw) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int rb = 32 * i + 8 * g + 4 * h;
                    const v4i s4 = *reinterpret_cast<const v4i*>(S + r0 + rb);
#pragma unroll
                    for (int vv = 0; vv < 4; ++vv) {
                        const uint32_t off = (uint32_t)(rb + vv) * (uint32_t)N + (uint32_t)l32;
#pragma unroll
                        for (int t = 0; t < TN; ++t) {
                            int32_t* at = aw + 32 * t;
                            at[off] = acc[i][t][4 * g + vv] - s4[vv];
                        }
                    }
                }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int rl = r0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
            const int row = m0 + rl;
            if (row >= M) continue;
            const float s = sc[rl];
            const int sm = S[rl];
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const int col = col_w + 32 * t + l32;
                if (col >= N) continue;
                const int a = acc[i][t][v] - sm;
                const int64_t o = (int64_t)row * N + col;
                if (y) y[o] = (float)a * s;
                if (acc_out) acc_out[o] = a;
            }
        }
    }
}

}  // namespace bl
