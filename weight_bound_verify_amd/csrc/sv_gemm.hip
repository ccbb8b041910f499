// q8b32 skinny matmul for gfx950: int8 rows with per-block-32 fp16 scales against S <= 64
// fp16 activation rows, fp32 accumulation, one pass over the weights.
//
// Contraction (pages: "Riding Apple's pipelined GPU engine", quantization on the GPU
// delegate -- linear per-block-32 int8; "Stream C - Speculative decoding", C1 substrate map
// and the delta -- all-position logits of the S = K+1 window, batched per-row argmax):
//   L[s, v] = sum_b f32(scale[v, b]) * sum_{k in block b} f32(q[v, k]) * f32(x[s, k])
//
// Mapping onto v_mfma_f32_16x16x32_f16 (one instruction = one 32-wide quantization block):
//   B operand (32 x 16) = the block of 16 weight rows; lane l holds row l%16, codes
//                         8*(l/16) .. +7 of the block, converted exactly to fp16.
//   A operand (16 x 32) = the matching block of 16 window rows (zeros past S), held in
//                         registers for the whole launch.
//   D (16 x 16) fp32    = lane l holds window rows 4*(l/16) .. +3 of weight row l%16, so the
//                         block scale of that weight row multiplies all four in fp32:
//                         acc += scale * D.  The sum over one block is exact (integer codes
//                         times fp16 values); only the cross-block accumulation rounds.
// A workgroup owns 16 weight rows at a time; its NW waves split the hidden axis, each
// holding its share of the window rows in registers, and reduce through LDS in a fixed
// order (deterministic).  The head epilogue keeps a running (value, lowest index) argmax
// per window row; only 8 bytes per (row, workgroup) leave the kernel.
#include "sv_device.h"
#include "sv_internal.h"

#include <climits>
#include <cmath>

namespace sv {

namespace {

int g_nw_override = 0;       // 0 = choose
int g_grid_override = 0;     // 0 = choose

template <int MT, int NBW, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void q8b32_kernel(GemmArgs a) {
    constexpr int NACC = (EPI == EPI_GATEUP) ? 2 : 1;
    __shared__ f32x4 red[2][NW][NACC * MT][kWave];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;       // weight row within the tile / window row within A
    const int g = lane >> 4;       // 8-code group within the block

    // hidden-axis range of this workgroup (ksplit) and of this wave
    const int ks = blockIdx.y;
    const int kb0 = (int)((long long)a.nb * ks / a.ksplit);
    const int kb1 = (int)((long long)a.nb * (ks + 1) / a.ksplit);
    const int nbk = kb1 - kb0;
    const int bw0 = kb0 + (int)((long long)nbk * wave / NW);
    const int nbw = kb0 + (int)((long long)nbk * (wave + 1) / NW) - bw0;

    // window rows for this wave's blocks, kept in registers
    f16x8 hid[NBW][MT];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int s = mt * 16 + n;
            f16x8 h = {};
            if (i < nbw && s < a.S)
                h = *reinterpret_cast<const f16x8*>(a.x + (size_t)s * a.H + (size_t)(bw0 + i) * kBlock + g * 8);
            hid[i][mt] = h;
        }
    }

    float best_v[MT][4];
    int best_i[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) { best_v[mt][r] = -INFINITY; best_i[mt][r] = INT_MAX; }

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    int buf = 0;
    for (int it = blockIdx.x; it < a.nitems; it += gridDim.x) {
        const int row0 = it * kTileRows;
        const int row = min(row0 + n, a.V - 1);        // tail rows re-read the last row; masked below

        u32x2 wv[NACC][NBW];
        uint16_t sv[NACC][NBW];
        {
            const int8_t* wp = a.w0 + (size_t)row * a.H + (size_t)bw0 * kBlock + g * 8;
            const uint16_t* sp = a.s0 + (size_t)row * a.nb + bw0;
#pragma unroll
            for (int i = 0; i < NBW; ++i)
                if (i < nbw) {
                    wv[0][i] = *reinterpret_cast<const u32x2*>(wp + i * kBlock);
                    sv[0][i] = sp[i];
                }
        }
        if constexpr (NACC == 2) {
            const int8_t* wp = a.w1 + (size_t)row * a.H + (size_t)bw0 * kBlock + g * 8;
            const uint16_t* sp = a.s1 + (size_t)row * a.nb + bw0;
#pragma unroll
            for (int i = 0; i < NBW; ++i)
                if (i < nbw) {
                    wv[NACC - 1][i] = *reinterpret_cast<const u32x2*>(wp + i * kBlock);
                    sv[NACC - 1][i] = sp[i];
                }
        }

        f32x4 acc[NACC][MT];
#pragma unroll
        for (int c = 0; c < NACC; ++c)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[c][mt] = zero;

#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            if (i < nbw) {
#pragma unroll
                for (int c = 0; c < NACC; ++c) {
                    const f16x8 b = i8x8_to_f16x8(wv[c][i]);
                    const float sc = h2f(sv[c][i]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(hid[i][mt], b, zero, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[c][mt][r] = __builtin_fmaf(sc, t[r], acc[c][mt][r]);
                    }
                }
            }
        }

#pragma unroll
        for (int c = 0; c < NACC; ++c)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[buf][wave][c * MT + mt][lane] = acc[c][mt];
        __syncthreads();

        if (wave == 0) {
            f32x4 tot[NACC][MT];
#pragma unroll
            for (int c = 0; c < NACC; ++c)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    f32x4 t = red[buf][0][c * MT + mt][lane];
#pragma unroll
                    for (int w = 1; w < NW; ++w) t += red[buf][w][c * MT + mt][lane];
                    tot[c][mt] = t;
                }
            const int v = row0 + n;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = mt * 16 + g * 4 + r;
                    if (s < a.S && v < a.V) {
                        const size_t o = (size_t)s * a.V + v;
                        if (a.ksplit > 1) {
                            const size_t po = (size_t)ks * a.S * a.V + o;
                            a.kpart0[po] = tot[0][mt][r];
                            if constexpr (NACC == 2) a.kpart1[po] = tot[NACC - 1][mt][r];
                        } else if constexpr (EPI == EPI_HEAD) {
                            const float val = tot[0][mt][r];
                            if (a.logits) a.logits[o] = val;
                            if (val > best_v[mt][r]) { best_v[mt][r] = val; best_i[mt][r] = v; }
                        } else if constexpr (EPI == EPI_STORE) {
                            float val = tot[0][mt][r];
                            if (a.residual) val += h2f(a.residual[o]);
                            a.y[o] = f2h(val);
                        } else {
                            const float gg = tot[0][mt][r];
                            const float uu = tot[NACC - 1][mt][r];
                            a.y[o] = f2h(gg / (1.0f + expf(-gg)) * uu);
                        }
                    }
                }
        }
        buf ^= 1;
    }

    if constexpr (EPI == EPI_HEAD) {
        if (a.ksplit == 1 && wave == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float bv = best_v[mt][r];
                    int bi = best_i[mt][r];
                    argmax_group<16>(bv, bi);
                    const int s = mt * 16 + g * 4 + r;
                    if (n == 0 && s < a.S) {
                        a.part_val[(size_t)s * kGridMax + blockIdx.x] = bv;
                        a.part_idx[(size_t)s * kGridMax + blockIdx.x] = bi;
                    }
                }
        }
    }
}

// ksplit > 1: sum the partial sums in split order, then apply the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void combine_kernel(GemmArgs a) {
    const int s = blockIdx.y;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int v = blockIdx.x * 256 + threadIdx.x; v < a.V; v += gridDim.x * 256) {
        const size_t o = (size_t)s * a.V + v;
        const size_t plane = (size_t)a.S * a.V;
        float t0 = a.kpart0[o];
        for (int k = 1; k < a.ksplit; ++k) t0 += a.kpart0[k * plane + o];
        if constexpr (EPI == EPI_HEAD) {
            if (a.logits) a.logits[o] = t0;
            if (t0 > bv) { bv = t0; bi = v; }
        } else if constexpr (EPI == EPI_STORE) {
            if (a.residual) t0 += h2f(a.residual[o]);
            a.y[o] = f2h(t0);
        } else {
            float t1 = a.kpart1[o];
            for (int k = 1; k < a.ksplit; ++k) t1 += a.kpart1[k * plane + o];
            a.y[o] = f2h(t0 / (1.0f + expf(-t0)) * t1);
        }
    }
    if constexpr (EPI == EPI_HEAD) {
        __shared__ float sv_[4];
        __shared__ int si_[4];
        argmax_group<64>(bv, bi);
        if ((threadIdx.x & 63) == 0) { sv_[threadIdx.x >> 6] = bv; si_[threadIdx.x >> 6] = bi; }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < 4; ++w)
                if (better(sv_[w], si_[w], bv, bi)) { bv = sv_[w]; bi = si_[w]; }
            a.part_val[(size_t)s * kGridMax + blockIdx.x] = bv;
            a.part_idx[(size_t)s * kGridMax + blockIdx.x] = bi;
        }
    }
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const float* pv, const int* pi, int nparts,
                                                           int* argmax) {
    const int s = blockIdx.x;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int p = threadIdx.x; p < nparts; p += 256) {
        const float v = pv[(size_t)s * kGridMax + p];
        const int i = pi[(size_t)s * kGridMax + p];
        if (better(v, i, bv, bi)) { bv = v; bi = i; }
    }
    __shared__ float sv_[4];
    __shared__ int si_[4];
    argmax_group<64>(bv, bi);
    if ((threadIdx.x & 63) == 0) { sv_[threadIdx.x >> 6] = bv; si_[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w)
            if (better(sv_[w], si_[w], bv, bi)) { bv = sv_[w]; bi = si_[w]; }
        argmax[s] = bi;
    }
}

typedef void (*KernelFn)(GemmArgs);

// Instantiated (MT, NBW, NW) shapes: all compile without register spills on gfx950
// (1024-thread workgroups are limited to 128 VGPRs, so NW = 16 only with small NBW).
struct Shape { int mt, nbw, nw; };
constexpr Shape kShapes[] = {
    {1, 4, 4}, {1, 8, 4}, {1, 16, 4}, {1, 4, 8}, {1, 8, 8}, {1, 16, 8}, {1, 4, 16}, {1, 8, 16},
    {2, 4, 4}, {2, 8, 4}, {2, 4, 8}, {2, 8, 8},
    {4, 2, 4}, {4, 4, 4}, {4, 2, 8},
};

template <int EPI>
KernelFn pick(const GemmCfg& c) {
#define SV_SHAPE(MT, NBW, NW) \
    if (c.mt == MT && c.nbw == NBW && c.nw == NW) return q8b32_kernel<MT, NBW, NW, EPI>;
    SV_SHAPE(1, 4, 4) SV_SHAPE(1, 8, 4) SV_SHAPE(1, 16, 4) SV_SHAPE(1, 4, 8) SV_SHAPE(1, 8, 8)
    SV_SHAPE(1, 16, 8) SV_SHAPE(1, 4, 16) SV_SHAPE(1, 8, 16)
    if constexpr (EPI == EPI_HEAD) {
        SV_SHAPE(2, 4, 4) SV_SHAPE(2, 8, 4) SV_SHAPE(2, 4, 8) SV_SHAPE(2, 8, 8)
        SV_SHAPE(4, 2, 4) SV_SHAPE(4, 4, 4) SV_SHAPE(4, 2, 8)
    }
#undef SV_SHAPE
    return nullptr;
}

// Smallest instantiated NBW >= need for (mt, nw); 0 if none.
int bucket(int need, int mt, int nw) {
    int best = 0;
    for (const Shape& sh : kShapes)
        if (sh.mt == mt && sh.nw == nw && sh.nbw >= need && (best == 0 || sh.nbw < best)) best = sh.nbw;
    return best;
}

}  // namespace

void set_tuning(int waves_per_group, int max_groups) {
    g_nw_override = waves_per_group;
    g_grid_override = max_groups;
}

namespace {

bool try_config(int rows, int H, int S, int nw_fixed, GemmCfg& c) {
    c.mt = S <= 16 ? 1 : (S <= 32 ? 2 : 4);
    const int nb = H / kBlock;
    const int pref[3] = {8, 16, 4};
    for (int ks = 1; ks <= nb; ++ks) {
        const int nbk = (nb + ks - 1) / ks;
        for (int t = 0; t < 3; ++t) {
            const int nw = nw_fixed ? nw_fixed : (nb < 32 ? 4 : pref[t]);
            const int b = bucket((nbk + nw - 1) / nw, c.mt, nw);
            if (b) {
                c.nw = nw;
                c.nbw = b;
                c.ksplit = ks;
                const int items = (rows + kTileRows - 1) / kTileRows;
                const int cap = g_grid_override ? g_grid_override : 1024;
                c.grid = items < cap ? items : cap;
                if (c.grid > kGridMax) c.grid = kGridMax;
                if (c.grid < 1) c.grid = 1;
                return true;
            }
            if (nw_fixed || nb < 32) break;
        }
    }
    return false;
}

}  // namespace

GemmCfg gemm_config(int rows, int H, int S) {
    GemmCfg c{};
    if (g_nw_override && try_config(rows, H, S, g_nw_override, c)) return c;
    try_config(rows, H, S, 0, c);       // always succeeds: (mt, smallest nbw, 4 waves) exists
    return c;
}

size_t head_workspace_bytes(int V, int H, int S) {
    const GemmCfg c = gemm_config(V, H, S);
    size_t b = (size_t)8 * S * kGridMax;
    if (c.ksplit > 1) b += (size_t)4 * c.ksplit * S * V;
    return b;
}

size_t stack_workspace_bytes(int N, int K, int S, bool gateup) {
    const GemmCfg c = gemm_config(N, K, S);
    if (c.ksplit == 1) return 0;
    return (size_t)4 * c.ksplit * S * N * (gateup ? 2 : 1);
}

hipError_t launch_q8b32(int epi, const GemmCfg& cfg, const GemmArgs& a, hipStream_t stream) {
    KernelFn fn = nullptr;
    if (epi == EPI_HEAD) fn = pick<EPI_HEAD>(cfg);
    else if (epi == EPI_STORE) fn = pick<EPI_STORE>(cfg);
    else fn = pick<EPI_GATEUP>(cfg);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, dim3(cfg.grid, cfg.ksplit), dim3(cfg.nw * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || cfg.ksplit == 1) return e;
    const int cg = (a.V + 255) / 256 < 256 ? (a.V + 255) / 256 : 256;
    if (epi == EPI_HEAD)
        hipLaunchKernelGGL(combine_kernel<EPI_HEAD>, dim3(cg, a.S), dim3(256), 0, stream, a);
    else if (epi == EPI_STORE)
        hipLaunchKernelGGL(combine_kernel<EPI_STORE>, dim3(cg, a.S), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(combine_kernel<EPI_GATEUP>, dim3(cg, a.S), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_argmax_final(const float* pv, const int* pi, int nparts, int S, int* argmax,
                               hipStream_t stream) {
    hipLaunchKernelGGL(argmax_final_kernel, dim3(S), dim3(256), 0, stream, pv, pi, nparts, argmax);
    return hipGetLastError();
}

}  // namespace sv
